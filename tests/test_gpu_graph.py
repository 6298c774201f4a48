"""The one-launch step captured into a HIP graph (launch amortisation across layers).

The library enqueues only kernels on the caller's stream (its workspace counters are
cleared by a kernel, never by a memset), so a multi-layer step can be captured once
and replayed.  Each replay re-appends the same rows at the same positions, so every
replay must reproduce the eager step bit for bit: outputs and whole caches.  Replays
are separated by unrelated eager work and synchronisations.
"""
import pytest
import torch

import decode_attention_append_amd as da
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, flush=True)


@pytest.mark.parametrize("B,q_len,Hq,Hkv,S,seq_pos,variant,merge", [
    (2, 1, 16, 8, 700, [699, 345], None, None),            # vector ALU, merge in the launch
    # vector-ALU long chunks (128 units, 2 rows): one chunk per sequence or
    # several, merged in the launch
    (16, 1, 16, 8, 3000, [2999 - 181 * i for i in range(16)], None, None),
    (2, 1, 64, 8, 3000, [2999, 1537], None, "launch"),     # MFMA, merge in the launch
    (2, 1, 64, 8, 3000, [2999, 1537], None, None),         # MFMA, separate merge: two launches
    (2, 4, 32, 4, 2100, [2096, 777], None, None),          # MFMA, 32 rows, causal, separate merge
    (2, 2, 32, 4, 900, [898, 250], "valu", None),          # forced 16-row VALU: three launches
])
def test_graph_replays_match_eager(B, q_len, Hq, Hkv, S, seq_pos, variant, merge):
    layers = 3
    _say("graph", B, q_len, Hq, Hkv, S, seq_pos, variant, merge)
    cases = [gu.make_case(B, q_len, Hq, Hkv, S, seq_pos, seed=100 + l) for l in range(layers)]
    p = da.problem_for(cases[0]["q"], cases[0]["k_cache"], variant=variant, merge=merge)
    ws = da.new_workspace(p)

    # eager reference on copies
    ref_out, ref_k, ref_v = [], [], []
    for c in cases:
        e = dict(c, k_cache=c["k_cache"].clone(), v_cache=c["v_cache"].clone())
        ref_out.append(gu.run_step(p, e, ws=ws))
        ref_k.append(e["k_cache"])
        ref_v.append(e["v_cache"])
    torch.cuda.synchronize()

    outs = [torch.empty_like(c["q"]) for c in cases]

    def step():
        for c, o in zip(cases, outs):
            da.decode_step(p, c["q"], c["k_cache"], c["v_cache"], c["k_new"], c["v_new"], c["seq_pos"], ws, o)

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

    junk = torch.randn(1024, 1024, device="cuda")
    for rep in range(4):
        for o in outs:
            o.zero_()
        g.replay()
        torch.cuda.synchronize()
        for l in range(layers):
            assert torch.equal(outs[l], ref_out[l]), f"replay {rep}, layer {l}: output differs from eager"
            assert torch.equal(cases[l]["k_cache"], ref_k[l]) and torch.equal(cases[l]["v_cache"], ref_v[l])
        # unrelated eager work between replays, including the library's separate path
        junk = junk @ junk.t() / 1024.0
        e = dict(cases[0], k_cache=cases[0]["k_cache"].clone(), v_cache=cases[0]["v_cache"].clone())
        o2 = gu.run_step(p, e, path="separate")
        torch.cuda.synchronize()
        assert torch.isfinite(o2.float()).all()
