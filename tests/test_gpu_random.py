"""Seeded random problems through every path of the step, against the oracle.

Each case draws its shape and features together, so that combinations the
fixed-shape tests do not list get run too: batch 1-5, 1-8 KV heads, 1-16 query
heads per KV head (a sixth of the cases 16-40 sequences over 4-16 KV heads, at
least 128 (sequence, KV head) pairs, caches up to 1500 slots), q_len 1-8 (at most 32 rows), head_dim 128 or 256, bf16 or
fp16, contiguous caches or page pools of up to 3000 slots (a tenth of the cases
8192-20000 slots over 4 or 8 KV heads, long enough for the longest chunks and
their alignment), positions at the first slot, the last one or anywhere
between, the rotary embedding over 64, 128 or 256 dims, the output gate, the
kernel forced or automatic, fixed or balanced chunks, the merge in the launch,
separate or automatic, inputs of spread 0.25, 1 or 4 (the last a sharp
softmax, without a rotary table), and a custom softmax scale.  Every case runs the
three separate calls, da_decode_step as planned, and da_decode_step with the
merge forced into the launch where that changes the launches, and checks the
caches bit for bit (rotated K rows within one ulp plus the fp32 evaluation
slack) and the output elementwise
within 1e-2 + 1e-2 |oracle|.
"""
import numpy as np
import pytest
import torch

import decode_attention_append_amd as da
from decode_attention_append_amd.workloads import rope_freqs
from tests import gpu_util as gu
from tests.oracle_pins import bits
from tests.test_gpu_paged import make_paged

N_CASES = 128


def spec(i: int) -> dict:
    """The i-th case: a valid problem (the host planning test checks that it plans)."""
    rng = np.random.default_rng(7000 + i)
    while True:
        D = int(rng.choice([128, 256], p=[0.7, 0.3]))
        Hkv = int(rng.choice([1, 2, 4, 8]))
        G = int(rng.choice([1, 2, 4, 8, 16]))
        q_len = int(rng.choice([1, 1, 1, 2, 3, 4, 8]))
        if G * q_len <= 32:
            break
    rows = G * q_len
    B = int(rng.integers(1, 6))
    mode = rng.random()
    long_ctx = mode < 0.1  # chunks long enough for the 2048-key alignment
    many = 0.1 <= mode < 0.25  # at least 128 (sequence, KV head) pairs: long VALU chunks, merge rules
    paged = bool(rng.random() < 0.3)
    if long_ctx:
        B, Hkv = int(rng.integers(1, 5)), int(rng.choice([4, 8]))
        G = min(G, 32 // q_len, 8)
        rows = G * q_len
    elif many:
        B, Hkv = int(rng.integers(16, 41)), int(rng.choice([4, 8, 16]))
        G = min(G, 4)
        B = max(B, -(-128 // Hkv))
        rows = G * q_len
    hi = 1500 if many else 3000
    if paged:
        pps = int(rng.integers(512, 1251)) if long_ctx else int(rng.integers(1, hi // 16 + 1))
        S = 16 * pps
    else:
        pps = 0
        S = int(rng.integers(8192, 20001)) if long_ctx else int(rng.integers(q_len, hi + 1))
    if S < q_len:  # one page shorter than a verify batch
        pps, S = 1, 16
    sp = []
    for _ in range(B):
        u = rng.random()
        sp.append(0 if u < 0.15 else S - q_len if u < 0.3 else int(rng.integers(0, S - q_len + 1)))
    variant = None
    u = rng.random()
    if u < 0.15 and D == 128 and rows <= 16:
        variant = "valu"
    elif u < 0.3:
        variant = "mfma"
    rope_dim, theta = None, 0.0
    if rng.random() < 0.3 and not (variant == "valu" and rows > 8):
        rope_dim = int(rng.choice([w for w in (64, 128, 256) if w <= D]))
        theta = float(rng.choice([1.0e4, 1.0e6, 1.0e7]))
    gate = bool(rng.random() < 0.3)
    chunk = 0 if rng.random() < 0.8 else 64 * int(rng.integers(1, 17))
    merge = [None, None, None, "launch", "separate"][int(rng.integers(0, 5))]
    dtype = "bf16" if rng.random() < 0.5 else "fp16"
    # inputs N(0, 1) times this (4: scores of spread 16, a sharp softmax); a softmax
    # scale other than 1/sqrt(head_dim) in a fifth of the cases.  A rotated q or K
    # element may round either way at a 16-bit boundary (the rotation is an fp32
    # evaluation); at spread 4 such a last-bit difference moves a score by up to
    # about 0.2 and a sharp softmax's output past the tolerance, so the sharp cases
    # run without a rotary table.
    data = float(rng.choice([1.0, 1.0, 1.0, 4.0, 0.25]))
    if rope_dim and data > 1.0:
        data = 1.0
    scale = float(rng.uniform(0.02, 0.3)) if rng.random() < 0.2 else 0.0
    return dict(B=B, q_len=q_len, Hq=G * Hkv, Hkv=Hkv, D=D, S=S, pps=pps, seq_pos=sp, dtype=dtype,
                variant=variant, rope_dim=rope_dim, theta=theta, gate=gate, chunk=chunk, merge=merge,
                data=data, scale=scale, seed=100 + i)


def test_random_cases_plan():
    """Host only: every case is a problem the library plans (no GPU needed)."""
    for i in range(N_CASES):
        s = spec(i)
        p = da.problem(s["B"], s["q_len"], s["Hq"], s["Hkv"], s["D"], s["S"], s["dtype"], scale=s["scale"],
                       chunk_tokens=s["chunk"], variant=s["variant"], merge=s["merge"])
        if s["rope_dim"]:
            p.rope_freqs, p.rope_dim = 0x1000, s["rope_dim"]
        if s["gate"]:
            p.out_gate = 0x2000
        if s["pps"]:
            p.page_size, p.pages_per_seq, p.n_pages, p.block_table = 16, s["pps"], s["B"] * s["pps"] + 5, 0x3000
        pl = da.plan_attention(p)
        assert pl["rows"] == s["Hq"] // s["Hkv"] * s["q_len"], s
        assert max(s["seq_pos"]) + s["q_len"] <= s["S"] and min(s["seq_pos"]) >= 0, s


def case_inputs(s: dict):
    """(device inputs, rotary table or None, problem) of case ``s``."""
    dt = torch.bfloat16 if s["dtype"] == "bf16" else torch.float16
    if s["pps"]:
        inp = make_paged(s["B"], s["q_len"], s["Hq"], s["Hkv"], s["pps"], s["seq_pos"], dt, seed=s["seed"],
                         scale=s["data"], head_dim=s["D"], gate=s["gate"])
    else:
        inp = gu.make_case(s["B"], s["q_len"], s["Hq"], s["Hkv"], s["S"], s["seq_pos"], dt, seed=s["seed"],
                           scale=s["data"], head_dim=s["D"], gate=s["gate"])
    freqs = rope_freqs(s["rope_dim"], s["theta"], "cuda") if s["rope_dim"] else None
    p = da.problem_for(inp["q"], inp["k_cache"], scale=s["scale"], chunk_tokens=s["chunk"], variant=s["variant"],
                       rope_freqs=freqs, block_table=inp.get("block_table"), rope_dim=s["rope_dim"] or 0,
                       out_gate=inp.get("out_gate"), merge=s["merge"])
    return inp, freqs, p


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(N_CASES))
def test_random_problem(i):
    s = spec(i)
    print("[case] random", i, s, flush=True)
    inp, freqs, p = case_inputs(s)
    gu.check_full(p, inp, freqs=freqs)


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(0, N_CASES, 4))
def test_random_decode_loop(i):
    """Every fourth case as a decode loop: four da_decode_step calls through one
    workspace, positions advancing by q_len, fresh q, new rows and gate each step,
    each step checked against the oracle from the caches the step before left."""
    s = spec(i)
    inp, freqs, p = case_inputs(s)
    ws = da.new_workspace(p)
    gen = torch.Generator(device="cpu").manual_seed(s["seed"])
    sp = np.asarray(s["seq_pos"], dtype=np.int32)
    for it in range(4):
        if it:
            sp = np.minimum(sp + s["q_len"], s["S"] - s["q_len"]).astype(np.int32)
            for k in ("q", "k_new", "v_new", "out_gate"):
                if k in inp:
                    inp[k].copy_(torch.randn(inp[k].shape, generator=gen).to(inp[k].dtype))
            inp["seq_pos"].copy_(torch.as_tensor(sp))
        print("[case] random loop", i, "step", it, sp.tolist(), flush=True)
        gu.check_full(p, inp, freqs=freqs, paths=("step",), ws=ws)


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(2, N_CASES, 8))
def test_random_contract_breaking(i):
    """Every eighth case with about a third of its sequences (at least one) given a
    position that breaks the contract (negative, or past max_seq - q_len): through the
    separate calls and da_decode_step, those sequences' cache rows stay untouched and
    their output rows are NaN, and the others match the oracle run on them alone."""
    s = spec(i)
    rng = np.random.default_rng(50000 + i)
    B, q_len, S = s["B"], s["q_len"], s["S"]
    bad = sorted(int(b) for b in rng.choice(B, max(1, B // 3), replace=False))
    sp = list(s["seq_pos"])
    for b in bad:
        sp[b] = int(rng.choice([-1, -7, S - q_len + 1, S, S + 1000]))
    s = dict(s, seq_pos=sp)
    good = np.asarray([b for b in range(B) if b not in bad], dtype=np.int64)
    print("[case] random contract", i, "bad", bad, s, flush=True)
    inp, freqs, p = case_inputs(s)
    dt = gu.odt(inp["q"].dtype)
    spa = np.asarray(sp, dtype=np.int32)
    bt = inp.get("block_table")
    bt = None if bt is None else bt.cpu().numpy()
    kc0, vc0 = bits(inp["k_cache"]), bits(inp["v_cache"])
    kn_all = bits(inp["k_new"])
    k_ref, v_ref = kc0.copy(), vc0.copy()
    new = np.zeros(kc0.shape[:3], bool)
    ref = None
    if good.size:
        spg = spa[good]
        kn, vn, qb = kn_all[good], bits(inp["v_new"])[good], bits(inp["q"])[good]
        if freqs is not None:
            fr = freqs.cpu().numpy()
            pos = spg[:, None, None] + np.arange(q_len, dtype=np.int32)[None, :, None]
            kn = gu.oracle.rope_rows(kn, np.broadcast_to(pos, kn.shape[:3]), fr, dt)
            qb = gu.oracle.rope_q(qb, spg, fr, dt)
        if bt is None:
            k_ref[good], v_ref[good] = gu.oracle.kv_append(kc0[good], vc0[good], kn, vn, spg)
            kc, vc = k_ref[good], v_ref[good]
        else:
            k_ref, v_ref = gu.oracle.kv_append_paged(kc0, vc0, kn, vn, spg, np.ascontiguousarray(bt[good]))
            kc = gu.oracle.gather_paged(k_ref, np.ascontiguousarray(bt[good]))
            vc = gu.oracle.gather_paged(v_ref, np.ascontiguousarray(bt[good]))
        ref = gu.oracle.gqa_decode(qb, kc, vc, spg, dt, scale=p.scale if p.scale > 0 else None)
        if "out_gate" in inp:
            ref = gu.oracle.output_gate(ref, np.ascontiguousarray(bits(inp["out_gate"])[good]), dt)
        for b in good:
            for t in range(spa[b], spa[b] + q_len):
                if bt is None:
                    new[b, :, t] = True
                else:
                    new[bt[b, t // 16], :, t % 16] = True
    for path in ("separate", "step"):
        run = dict(inp, k_cache=inp["k_cache"].clone(), v_cache=inp["v_cache"].clone())
        out = gu.run_step(p, run, path=path)
        torch.cuda.synchronize()
        kg = bits(run["k_cache"])
        assert np.array_equal(bits(run["v_cache"]), v_ref), f"{path}: v cache"
        if freqs is None:
            assert np.array_equal(kg, k_ref), f"{path}: k cache"
        else:
            gu.check_rotated_k(kg, k_ref, new, kn_all, spa, q_len, 2 * freqs.numel(), dt, bt, path)
        o = out.float().cpu()
        assert torch.isnan(o[bad]).all(), f"{path}: rows of contract-breaking sequences are not NaN"
        if ref is not None:
            gu.compare_out(out[good.tolist()], ref, f"{path}: the other sequences")


def _same_bits(a, b):
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(1, N_CASES, 8))
def test_random_graph_replays(i):
    """Every eighth case captured into a HIP graph (one da_decode_step): three
    replays, with unrelated eager work and synchronisations between them, each
    reproduce the eager step bit for bit, output and whole caches (a replay appends
    the same rows at the same positions again)."""
    s = spec(i)
    print("[case] random graph", i, s, flush=True)
    inp, _, p = case_inputs(s)
    ws = da.new_workspace(p)
    e = dict(inp, k_cache=inp["k_cache"].clone(), v_cache=inp["v_cache"].clone())
    ref_out = gu.run_step(p, e, ws=ws)
    torch.cuda.synchronize()
    out = torch.empty_like(inp["q"])

    def step():
        da.decode_step(p, inp["q"], inp["k_cache"], inp["v_cache"], inp["k_new"], inp["v_new"], inp["seq_pos"],
                       ws, out)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # the first run outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    junk = torch.randn(512, 512, device="cuda")
    for rep in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert _same_bits(out, ref_out), f"replay {rep}: output differs from the eager step"
        assert _same_bits(inp["k_cache"], e["k_cache"]) and _same_bits(inp["v_cache"], e["v_cache"]), \
            f"replay {rep}: caches differ from the eager step"
        junk = junk @ junk.t() / 512.0
        torch.cuda.synchronize()
