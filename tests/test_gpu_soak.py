"""Soak of the in-launch merge: one-launch steps whose last chunk of each
(sequence, KV head) merges partials that other workgroups, on any XCD, wrote in
the same launch.  A step captured into a HIP graph is replayed 1000 times; the
merge order is fixed, so every replay must reproduce the first one bit for bit
(outputs and whole caches), and the test stops at the first replay that does
not.  A stale partial read by a merge would show up as a changed output.  The two
matrix-core workloads force the merge into the launch (with 32 heads their automatic
plan merges in a separate combine launch)."""
import pytest
import torch

import decode_attention_append_amd as da
from decode_attention_append_amd.workloads import WORKLOADS, make_layer
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

REPLAYS = 1000


def _case(name):
    if name in WORKLOADS:
        w = WORKLOADS[name]
        L = make_layer(w, 0, torch.device("cuda"))
        return L, da.problem(w.batch, w.q_len, w.n_q_heads, w.n_kv_heads, w.head_dim, w.max_seq, w.dtype,
                             out_gate=L.get("out_gate"), merge="launch")
    # a 4-wave vector-ALU shape merged in the launch: batch 1, 16 MHA heads, 4k context
    # (forced: the automatic plan takes the matrix-core kernel for so few heads)
    L = gu.make_case(1, 1, 16, 16, 4096, [4095], dtype=torch.float16, seed=5)
    return L, da.problem_for(L["q"], L["k_cache"], variant="valu")


@pytest.mark.parametrize("name", ["gqa64x8_b4_ctx12k_16k", "valu_mha16_ctx4096",
                                  "qwen35_gqa16x2_d256_gated_b16_ctx8192_10l"])
def test_merge_replays_bit_identical(name):
    print(f"[case] soak {name}, {REPLAYS} replays", flush=True)
    L, p = _case(name)
    plan = da.plan_attention(p)
    assert plan["fused_combine"], plan
    ws = da.new_workspace(p)
    out = torch.empty_like(L["q"])

    def step():
        da.decode_step(p, L["q"], L["k_cache"], L["v_cache"], L["k_new"], L["v_new"], L["seq_pos"], ws, out)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    g.replay()
    torch.cuda.synchronize()
    first = out.clone()
    k0, v0 = L["k_cache"].clone(), L["v_cache"].clone()
    assert torch.isfinite(first.float()).all()
    for rep in range(1, REPLAYS):
        out.zero_()
        g.replay()
        same = torch.equal(out, first)
        if rep % 100 == 0 or not same:
            same = same and torch.equal(L["k_cache"], k0) and torch.equal(L["v_cache"], v0)
        assert same, f"{name}: replay {rep} differs from the first"
    torch.cuda.synchronize()
