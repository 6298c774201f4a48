"""Seeded synthetic inputs for the decode-attention step.

This module only draws random numbers and lays them out; it holds none of the
attention arithmetic.  Both the GPU library's tests/benchmark and the oracle's
checks take their inputs from here, so it is the one module the two sides share.

Recipe (one decode step; every tensor drawn from a ``torch.Generator`` seeded
per layer as ``seed * 1000 + layer``, in this order):

  q        [B, q_len, Hq, D]      N(0,1) * value_scale, drawn in the element dtype
  k_cache  [B, Hkv, S, D]         same
  v_cache  [B, Hkv, S, D]         same
  k_new    [B, q_len, Hkv, D]     same
  v_new    [B, q_len, Hkv, D]     same
  out_gate [B, q_len, Hq, D]      N(0,1), unscaled (gated workloads only; drawn last)

Integer draws come from a separate CPU generator seeded with ``seed``:
per-sequence context lengths (or positions) first, then the heavy-row mask
(``heavy_fraction`` of the K rows of the whole allocated cache and of ``k_new``
multiplied by ``heavy_factor``).  value_scale and heavy_factor are powers of
two, so scaling is exact in bf16/fp16.

The decode workloads restate the attention shapes of the Qwen decodes the
pages profile (Qwen3-0.6B 16:8 heads, Qwen1.5-MoE-A2.7B 16 MHA heads, a GQA-8
long context, a 4-token speculative verify, and the full-attention layers of
Qwen3.5-35B-A3B: 16:2 heads of 256 dims, rotary on a quarter of the dims and a
sigmoid output gate); no trained weights or prompts are involved, all values
are synthetic.  A workload with a rotary width takes its frequency table from
``rope_freqs`` at ``rope_theta``.
"""
from dataclasses import dataclass, field
from typing import Optional, Tuple

import torch

DTYPES = {"bf16": torch.bfloat16, "fp16": torch.float16}


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    q_len: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    dtype: str
    max_seq: int
    layers: int
    seed: int
    value_scale: float = 1.0
    seq_pos: Optional[int] = None                 # same slot for every sequence
    ctx_range: Optional[Tuple[int, int]] = None   # inclusive, context length after append
    pos_range: Optional[Tuple[int, int]] = None   # inclusive, seq_pos of the first new token
    heavy_fraction: float = 0.0
    heavy_factor: float = 8.0
    rope_dim: int = 0            # rotated leading dims (0: no rotary embedding in the step)
    rope_theta: float = 0.0
    gated: bool = False          # out *= sigmoid(out_gate)
    note: str = field(default="", compare=False)

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def rows(self) -> int:
        return self.group * self.q_len

    @property
    def torch_dtype(self):
        return DTYPES[self.dtype]

    @property
    def elem_bytes(self) -> int:
        return 2


WORKLOADS = {
    w.name: w
    for w in [
        Workload("qwen3_0p6b_b1_ctx512", batch=1, q_len=1, n_q_heads=16, n_kv_heads=8,
                 head_dim=128, dtype="bf16", max_seq=512, layers=1, seed=1001, seq_pos=511,
                 note="single layer, Qwen3-0.6B attention shape"),
        Workload("qwen15moe_mha16_b1_ctx4096_24l", batch=1, q_len=1, n_q_heads=16,
                 n_kv_heads=16, head_dim=128, dtype="fp16", max_seq=4096, layers=24,
                 seed=1002, seq_pos=4095,
                 note="24 independent layers, Qwen1.5-MoE-A2.7B attention shape (MHA)"),
        Workload("gqa16x8_b32_ctx8192_28l", batch=32, q_len=1, n_q_heads=16, n_kv_heads=8,
                 head_dim=128, dtype="bf16", max_seq=8192, layers=28, seed=1003,
                 value_scale=0.5, seq_pos=8191,
                 note="batched GQA decode, 28 layers, every sequence at context 8192"),
        Workload("gqa64x8_b4_ctx12k_16k", batch=4, q_len=1, n_q_heads=64, n_kv_heads=8,
                 head_dim=128, dtype="bf16", max_seq=16384, layers=1, seed=1004,
                 ctx_range=(12288, 16384),
                 note="long-context GQA ratio 8, ragged contexts"),
        Workload("verify4_gqa32x4_b8_pos2048_8188", batch=8, q_len=4, n_q_heads=32,
                 n_kv_heads=4, head_dim=128, dtype="bf16", max_seq=8192, layers=1,
                 seed=1005, pos_range=(2048, 8188), heavy_fraction=0.01, heavy_factor=8.0,
                 note="speculative verify of 4 draft tokens, causal inside the window"),
        Workload("qwen35_gqa16x2_d256_gated_b16_ctx8192_10l", batch=16, q_len=1, n_q_heads=16,
                 n_kv_heads=2, head_dim=256, dtype="fp16", max_seq=8192, layers=10, seed=1006,
                 ctx_range=(6144, 8192), rope_dim=64, rope_theta=1.0e7, gated=True,
                 note="Qwen3.5-35B-A3B full-attention layers: 16:2 heads of 256 dims, partial "
                      "rotary (64 dims), sigmoid output gate, ragged contexts"),
    ]
}

# The throughput workload: Hq16/Hkv8/d128 at context 8192.
BENCH_WORKLOAD = "gqa16x8_b32_ctx8192_28l"


def _integer_draws(w: Workload):
    """CPU-generator draws, in order: per-sequence positions, then heavy-row masks."""
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed)
    if w.seq_pos is not None:
        seq_pos = torch.full((w.batch,), w.seq_pos, dtype=torch.int32)
    elif w.ctx_range is not None:
        lo, hi = w.ctx_range
        ctx = torch.randint(lo, hi + 1, (w.batch,), generator=g, dtype=torch.int64)
        seq_pos = (ctx - w.q_len).to(torch.int32)
    else:
        lo, hi = w.pos_range
        seq_pos = torch.randint(lo, hi + 1, (w.batch,), generator=g,
                                dtype=torch.int64).to(torch.int32)
    km = nm = None
    if w.heavy_fraction > 0.0:
        km = torch.rand((w.batch, w.n_kv_heads, w.max_seq), generator=g) < w.heavy_fraction
        nm = torch.rand((w.batch, w.q_len, w.n_kv_heads), generator=g) < w.heavy_fraction
    return seq_pos, km, nm


def make_tensors(batch, q_len, n_q_heads, n_kv_heads, head_dim, max_seq, dtype, seed,
                 device="cpu", value_scale=1.0, gate=False):
    """q, k_cache, v_cache, k_new, v_new drawn N(0,1)*value_scale in ``dtype``; with
    ``gate`` also an N(0,1) out_gate like q, drawn after them."""
    tdt = DTYPES[dtype] if isinstance(dtype, str) else dtype
    g = torch.Generator(device=device)
    g.manual_seed(seed)

    def draw(*shape):
        t = torch.randn(shape, generator=g, device=device, dtype=tdt)
        if value_scale != 1.0:
            t.mul_(value_scale)
        return t

    q = draw(batch, q_len, n_q_heads, head_dim)
    k_cache = draw(batch, n_kv_heads, max_seq, head_dim)
    v_cache = draw(batch, n_kv_heads, max_seq, head_dim)
    k_new = draw(batch, q_len, n_kv_heads, head_dim)
    v_new = draw(batch, q_len, n_kv_heads, head_dim)
    if gate:
        return q, k_cache, v_cache, k_new, v_new, torch.randn(q.shape, generator=g, device=device, dtype=tdt)
    return q, k_cache, v_cache, k_new, v_new


def make_layer(w: Workload, layer: int = 0, device="cpu"):
    """All inputs of one layer of a workload: dict of tensors on ``device``."""
    t = make_tensors(w.batch, w.q_len, w.n_q_heads, w.n_kv_heads, w.head_dim, w.max_seq,
                     w.dtype, w.seed * 1000 + layer, device, w.value_scale, gate=w.gated)
    q, kc, vc, kn, vn = t[:5]
    seq_pos, km, nm = _integer_draws(w)
    if km is not None:
        kc[km.to(device)] *= w.heavy_factor
        kn[nm.to(device)] *= w.heavy_factor
    seq_pos = seq_pos.to(device)
    out = {"q": q, "k_cache": kc, "v_cache": vc, "k_new": kn, "v_new": vn, "seq_pos": seq_pos}
    if w.gated:
        out["out_gate"] = t[5]
    return out


def rope_freqs(head_dim: int = 128, theta: float = 1.0e6, device="cpu") -> torch.Tensor:
    """A rotary frequency table, theta^(-2j/head_dim) for j < head_dim/2, as float32: an
    input of the step like the page's precomputed freqs table (theta 1e6 is Qwen3's
    rope_theta, 1e4 Qwen1.5's).  For a partial rotary embedding pass the rotated width
    as ``head_dim``: the table then holds rope_dim/2 values theta^(-2j/rope_dim)."""
    j = torch.arange(0, head_dim, 2, dtype=torch.float64)
    return (theta ** (-j / head_dim)).to(torch.float32).to(device)
