"""GPU parity of the paged KV cache (page pools + block table) against the oracle.

The pools follow the paged-attention layout [pages][KV heads][16 tokens][D];
each sequence's pages are scattered over the pool by a random permutation, and
the pool's unused pages hold NaN/inf so a read through a wrong page shows up.
Whole pools must match the oracle's paged append bit for bit (rotated K rows
within one ulp plus the fp32 evaluation slack when a rotary table is given),
outputs within
|d| <= 1e-2 + 1e-2 |ref| of the oracle's attention over the gathered caches.
"""
import numpy as np
import pytest
import torch

import decode_attention_append_amd as da
from decode_attention_append_amd.workloads import make_tensors, rope_freqs
from tests import gpu_util as gu
from tests.oracle_pins import bits

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, flush=True)


def make_paged(B, q_len, Hq, Hkv, pps, seq_pos, dtype=torch.bfloat16, seed=0, spare=5, scale=1.0,
               head_dim=128, gate=False):
    """Pools of B * pps + spare pages; sequence pages are a random permutation; spare pages
    are poisoned.  With ``gate`` the case also holds an out_gate."""
    n_pages = B * pps + spare
    D = head_dim
    _, kp, vp, _, _ = make_tensors(1, 1, Hkv, Hkv, D, n_pages * 16, dtype, seed, "cuda", scale)
    t = make_tensors(B, q_len, Hq, Hkv, D, 16, dtype, seed + 1, "cuda", scale, gate=gate)
    q, kn, vn = t[0], t[3], t[4]
    # the [1, Hkv, n_pages * 16, D] draw regrouped as [n_pages, Hkv, 16, D] pages
    kp = kp.reshape(Hkv, n_pages, 16, D).transpose(0, 1).contiguous()
    vp = vp.reshape(Hkv, n_pages, 16, D).transpose(0, 1).contiguous()
    rng = np.random.default_rng(seed)
    perm = rng.permutation(n_pages).astype(np.int32)
    bt = perm[:B * pps].reshape(B, pps)
    for pg in perm[B * pps:]:
        kp[pg] = float("nan")
        vp[pg] = float("inf")
    out = {"q": q, "k_cache": kp, "v_cache": vp, "k_new": kn, "v_new": vn,
           "seq_pos": torch.as_tensor(np.asarray(seq_pos, np.int32)).cuda(),
           "block_table": torch.as_tensor(bt).cuda()}
    if gate:
        out["out_gate"] = t[5]
    return out


def check_paged(p, inp, path, freqs=None, rows=None):
    dt = gu.odt(inp["q"].dtype)
    bt = inp["block_table"].cpu().numpy()
    sp = inp["seq_pos"].cpu().numpy()
    kp0, vp0 = bits(inp["k_cache"]), bits(inp["v_cache"])
    kn = kn_raw = bits(inp["k_new"])
    qb = bits(inp["q"])
    if freqs is not None:
        fr = freqs.cpu().numpy()
        pos = sp[:, None, None] + np.arange(p.q_len, dtype=np.int32)[None, :, None]
        kn = gu.oracle.rope_rows(kn, np.broadcast_to(pos, kn.shape[:3]), fr, dt)
        qb = gu.oracle.rope_q(qb, sp, fr, dt)
    kp_ref, vp_ref = gu.oracle.kv_append_paged(kp0, vp0, kn, bits(inp["v_new"]), sp, bt)
    out = gu.run_step(p, inp, path=path)
    torch.cuda.synchronize()
    assert np.array_equal(bits(inp["v_cache"]), vp_ref), "v pool differs from the oracle's paged append"
    kg = bits(inp["k_cache"])
    if freqs is None:
        assert np.array_equal(kg, kp_ref), "k pool differs from the oracle's paged append"
    else:
        new = gu.appended_rows(kp_ref.shape, sp, p.q_len, bt)
        gu.check_rotated_k(kg, kp_ref, new, kn_raw, sp, p.q_len, 2 * freqs.numel(), dt, bt, "paged")
    kc, vc = gu.oracle.gather_paged(kp_ref, bt), gu.oracle.gather_paged(vp_ref, bt)
    if rows is None:
        ref = gu.oracle.gqa_decode(qb, kc, vc, sp, dt)
        return gu.compare_out(out, ref, f"{path}: paged")
    rows = np.asarray(rows, dtype=np.int32).reshape(-1, 3)
    ref = gu.oracle.gqa_decode_rows(qb, kc, vc, sp, rows, dt)
    o = out.cpu()
    return gu.compare_out(torch.stack([o[b, i, hq] for b, i, hq in rows]), ref, f"{path}: paged rows")


@pytest.mark.parametrize("path", gu.PATHS)
@pytest.mark.parametrize("B,q_len,Hq,Hkv,pps,seq_pos,dtype", [
    (3, 1, 16, 8, 40, [639, 17, 300], torch.bfloat16),          # vector ALU, 2 rows
    (2, 1, 16, 16, 64, [1023, 64], torch.float16),              # MHA fp16
    (2, 1, 64, 8, 190, [3039, 1537], torch.bfloat16),           # MFMA, 8 rows
    (2, 4, 32, 4, 132, [2108, 777], torch.bfloat16),            # MFMA, 32 rows, causal
    (2, 4, 8, 8, 45, [716, 61], torch.bfloat16),                # vector ALU, 4 draft tokens
    (2, 8, 4, 2, 32, [504, 3], torch.float16),                  # MFMA, q_len 8
])
def test_paged_shapes(B, q_len, Hq, Hkv, pps, seq_pos, dtype, path):
    _say("paged", B, q_len, Hq, Hkv, pps, seq_pos, dtype, path)
    inp = make_paged(B, q_len, Hq, Hkv, pps, seq_pos, dtype, seed=pps + B)
    p = da.problem_for(inp["q"], inp["k_cache"], block_table=inp["block_table"])
    check_paged(p, inp, path)


@pytest.mark.parametrize("path", gu.PATHS)
@pytest.mark.parametrize("chunk,variant", [(64, "valu"), (64, "mfma"), (128, "mfma"), (0, "valu")])
def test_paged_pages_across_chunks(chunk, variant, path):
    """Draft tokens straddling a page and a chunk boundary."""
    _say("paged straddle", chunk, variant, path)
    inp = make_paged(2, 4, 8, 8, 20, [62, 190], seed=chunk + 3)
    p = da.problem_for(inp["q"], inp["k_cache"], block_table=inp["block_table"], chunk_tokens=chunk,
                       variant=variant)
    check_paged(p, inp, path)


@pytest.mark.parametrize("path", gu.PATHS)
@pytest.mark.parametrize("B,Hq,Hkv,D,pps,seq_pos,chunk,pages,variant", [
    (2, 64, 8, 128, 257, [4095, 2600], 4096, 256, None),     # MFMA: one page per thread
    (2, 16, 2, 256, 257, [4095, 2600], 4096, 256, None),     # head_dim 256
    (2, 16, 8, 128, 257, [4095, 2600], 4096, 256, None),     # MFMA, 2 rows
    (2, 16, 8, 128, 257, [4095, 2600], 2048, 128, "valu"),   # vector ALU, 4 waves
    (16, 16, 8, 128, 400, [6300] + [211 * i + 5 for i in range(15)], 6304, 394, None),  # vector ALU, long chunks
    (16, 16, 8, 128, 512, [8191] + [211 * i + 5 for i in range(15)], 8192, 512, None),  # vector ALU, two pages per thread
])
def test_paged_long_chunks(B, Hq, Hkv, D, pps, seq_pos, chunk, pages, variant, path):
    """Chunks of up to one page per thread of the workgroup (two on the vector-ALU
    kernel's long chunks): each workgroup reads its chunk's page list into LDS once and
    takes every tile's or slab's page from there.  One requested work item gives every
    sequence its fewest, longest chunks."""
    _say("paged long chunks", B, Hq, Hkv, D, pps, chunk, path)
    inp = make_paged(B, 1, Hq, Hkv, pps, seq_pos, head_dim=D, seed=pps + D)
    p = da.problem_for(inp["q"], inp["k_cache"], block_table=inp["block_table"], work_items=1, variant=variant)
    assert max(ln for _, ln in da.chunk_layout(p, seq_pos)) == chunk
    assert -(-chunk // 16) == pages
    rng = np.random.default_rng(pps)
    rows = [(b, 0, int(h)) for b in range(min(B, 4)) for h in rng.choice(Hq, 4, replace=False)]
    check_paged(p, inp, path, rows=rows)


@pytest.mark.parametrize("path", gu.PATHS)
@pytest.mark.parametrize("Hq,Hkv,q_len", [(16, 8, 1), (32, 4, 4)])
def test_paged_with_rope(Hq, Hkv, q_len, path):
    _say("paged rope", Hq, Hkv, q_len, path)
    inp = make_paged(3, q_len, Hq, Hkv, 70, [1000, 63, 500], seed=Hq)
    freqs = rope_freqs(128, 1.0e6, "cuda")
    p = da.problem_for(inp["q"], inp["k_cache"], block_table=inp["block_table"], rope_freqs=freqs)
    check_paged(p, inp, path, freqs=freqs)


def test_paged_long_context_sampled():
    """A 64k-token sequence over 4096 scattered pages and a short one."""
    _say("paged long")
    inp = make_paged(2, 1, 16, 8, 4096, [65535, 3000], seed=9)
    p = da.problem_for(inp["q"], inp["k_cache"], block_table=inp["block_table"])
    rows = np.array([[0, 0, h] for h in range(16)] + [[1, 0, h] for h in range(0, 16, 5)])
    check_paged(p, inp, "step", rows=rows)


def test_paged_decode_loop():
    """Four one-launch steps on one pool and workspace, each sequence growing across pages."""
    B, q_len, Hq, Hkv, pps = 3, 2, 16, 8, 30
    inp = make_paged(B, q_len, Hq, Hkv, pps, [13, 200, 476], seed=11)
    p = da.problem_for(inp["q"], inp["k_cache"], block_table=inp["block_table"])
    ws = da.new_workspace(p)
    bt = inp["block_table"].cpu().numpy()
    kp, vp = bits(inp["k_cache"]), bits(inp["v_cache"])
    sp = inp["seq_pos"].cpu().numpy()
    gen = torch.Generator().manual_seed(12)
    for it in range(4):
        _say("paged loop", it, sp.tolist())
        if it:
            for k in ("q", "k_new", "v_new"):
                inp[k] = torch.randn(inp[k].shape, generator=gen).to(torch.bfloat16).cuda()
            inp["seq_pos"] = torch.as_tensor(sp).cuda()
        out = gu.run_step(p, inp, ws=ws)
        torch.cuda.synchronize()
        kp, vp = gu.oracle.kv_append_paged(kp, vp, bits(inp["k_new"]), bits(inp["v_new"]), sp, bt)
        assert np.array_equal(bits(inp["k_cache"]), kp) and np.array_equal(bits(inp["v_cache"]), vp)
        ref = gu.oracle.gqa_decode(bits(inp["q"]), gu.oracle.gather_paged(kp, bt), gu.oracle.gather_paged(vp, bt),
                                   sp, gu.oracle.BF16)
        gu.compare_out(out, ref, f"step {it}")
        sp = np.minimum(sp + q_len, pps * 16 - q_len).astype(np.int32)


@pytest.mark.parametrize("path", gu.PATHS)
@pytest.mark.parametrize("Hq,Hkv", [(16, 8), (64, 8)])
def test_paged_bad_block_table_entry_stays_in_the_pools(Hq, Hkv, path):
    """Sequence 0's block table names a page past the pool (and one below zero): no write
    lands outside its valid pages and sequence 1 is computed as usual."""
    _say("paged bad entry", Hq, Hkv, path)
    inp = make_paged(2, 1, Hq, Hkv, 10, [150, 100], seed=13)
    bt = inp["block_table"].clone()
    bt[0, 3] = 10_000
    bt[0, 9] = -3      # the page the new row of sequence 0 goes to
    inp["block_table"] = bt
    p = da.problem_for(inp["q"], inp["k_cache"], block_table=bt)
    kp0, vp0 = bits(inp["k_cache"]), bits(inp["v_cache"])
    out = gu.run_step(p, inp, path=path)
    torch.cuda.synchronize()
    good = inp["block_table"][1].cpu().numpy()
    kp, vp = bits(inp["k_cache"]), bits(inp["v_cache"])
    # only sequence 1's new slot changed
    changed = np.argwhere((kp != kp0).any(axis=(1, 3)))
    assert all(int(pg) == good[100 // 16] for pg, _ in changed), changed
    sub = lambda x: np.ascontiguousarray(x[1:2])  # noqa: E731
    bt1 = good[None, :]
    k_ref, v_ref = gu.oracle.kv_append_paged(kp0, vp0, sub(bits(inp["k_new"])), sub(bits(inp["v_new"])),
                                             np.array([100], np.int32), bt1)
    assert np.array_equal(kp, k_ref) and np.array_equal(vp, v_ref)
    ref = gu.oracle.gqa_decode(sub(bits(inp["q"])), gu.oracle.gather_paged(k_ref, bt1),
                               gu.oracle.gather_paged(v_ref, bt1), np.array([100], np.int32), gu.oracle.BF16)
    gu.compare_out(out[1:2], ref)
