"""The C-ABI library on the host: it loads, exports what the header declares, and
rejects bad arguments with the documented status before touching the GPU."""
import ctypes
import glob
import os
import re

import pytest

import decode_attention_append_amd as da

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"\b(da_[a-z_0-9]+)\s*\(", text))
    return sorted(names)


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("da_kv_append", "da_gqa_decode_attn", "da_gqa_decode_attn_combine",
              "da_workspace_bytes", "da_plan_attention", "da_status_str"):
        assert n in names


@pytest.mark.parametrize("name", declared_functions())
def test_library_exports(name):
    assert hasattr(da.lib, name), f"{name} declared in include/ but not exported"


def test_exports_match_binding_list():
    assert set(da.EXPORTS) <= set(declared_functions())


def P(**kw):
    base = dict(batch=2, q_len=1, n_q_heads=16, n_kv_heads=8, head_dim=128, max_seq=1024,
                dtype="bf16")
    base.update(kw)
    return da.problem(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(batch=0), da.DA_ERR_INVALID_ARG),
    (dict(q_len=0), da.DA_ERR_INVALID_ARG),
    (dict(n_q_heads=12, n_kv_heads=8), da.DA_ERR_INVALID_ARG),
    (dict(max_seq=0), da.DA_ERR_INVALID_ARG),
    (dict(q_len=9), da.DA_ERR_UNSUPPORTED),
    (dict(head_dim=64), da.DA_ERR_UNSUPPORTED),
    (dict(dtype=7), da.DA_ERR_UNSUPPORTED),
    (dict(n_q_heads=64, n_kv_heads=1, q_len=1), da.DA_ERR_UNSUPPORTED),  # 64 rows per KV head
    (dict(chunk_tokens=100), da.DA_ERR_INVALID_ARG),
    (dict(chunk_tokens=4096), da.DA_ERR_INVALID_ARG),
    (dict(q_len=8, max_seq=4), da.DA_ERR_INVALID_ARG),
    (dict(batch=1 << 19, n_q_heads=64, n_kv_heads=64, max_seq=64), da.DA_ERR_UNSUPPORTED),  # B * Hkv = 2^25
])
def test_plan_rejects(kw, status):
    p = P(**kw) if "dtype" not in kw or isinstance(kw["dtype"], str) else None
    if p is None:
        p = P()
        p.dtype = kw["dtype"]
    pl = da.Plan()
    assert da.lib.da_plan_attention(ctypes.byref(p), ctypes.byref(pl)) == status
    assert da.workspace_bytes(p) == 0


def test_plan_takes_the_largest_head_count():
    """B * Hkv just below 2^25 plans (the arrival counters' int32 offsets still fit)."""
    p = P(batch=(1 << 19) - 1, n_q_heads=64, n_kv_heads=64, max_seq=64)
    pl = da.Plan()
    assert da.lib.da_plan_attention(ctypes.byref(p), ctypes.byref(pl)) == da.DA_OK
    assert pl.workspace_bytes >= ((1 << 19) - 1) * 64 * 128


def test_plan_rejects_unknown_merge():
    for bad in (-1, 3):
        p = P()
        p.merge = bad
        assert da.lib.da_plan_attention(ctypes.byref(p), ctypes.byref(da.Plan())) == da.DA_ERR_INVALID_ARG


def test_plan_is_pure_and_sized():
    p = P(batch=32, max_seq=8192)
    a, b = da.plan_attention(p), da.plan_attention(p)
    assert a == b
    rows = 2
    assert a["balanced"] and a["variant"] == "valu"
    # long chunks aim at 256; slots and grid hold the most chunks of the plan for
    # uneven contexts, which aims at 1024 (over 8 KV heads: 128 per sequence)
    assert a["target_items"] == 256 and a["chunk_tokens"] == 8192
    assert a["n_chunks"] == 1024 // 8
    assert a["workspace_bytes"] >= 32 * 8 * a["n_chunks"] * rows * (128 + 2) * 4
    assert a["items"] >= 1024 + 32 * 8
    assert da.plan_attention(P(q_len=4, n_q_heads=32, n_kv_heads=4))["variant"] == "mfma"
    fixed = da.plan_attention(P(chunk_tokens=128))
    assert not fixed["balanced"] and fixed["chunk_tokens"] == 128 and fixed["n_chunks"] == 8
    assert fixed["items"] == 2 * 8 * 8
    assert da.plan_attention(P(work_items=77))["target_items"] == 77
    assert da.plan_attention(P(variant="mfma"))["variant"] == "mfma"


def test_plan_bounds():
    # the combine keeps one weight per chunk slot: never more than 2048 slots
    big = da.plan_attention(P(batch=1, n_q_heads=16, n_kv_heads=1, max_seq=1 << 21))
    assert big["n_chunks"] <= 2048 and big["chunk_tokens"] * 2048 >= (1 << 21)
    assert da.workspace_bytes(P(max_seq=(1 << 21) + 64)) == 0
    assert da.workspace_bytes(P(chunk_tokens=64, max_seq=64 * 2049)) == 0
    # forcing the vector-ALU kernel past its 16 rows is refused
    assert da.workspace_bytes(P(n_q_heads=32, n_kv_heads=1, variant="valu")) == 0


def test_null_and_misaligned_pointers_rejected_before_launch():
    p = P()
    buf = (ctypes.c_uint8 * 64)()
    good = ctypes.addressof(buf) + (-ctypes.addressof(buf)) % 16
    assert da.lib.da_kv_append(ctypes.byref(p), None, good, good, good, good, None) == da.DA_ERR_INVALID_ARG
    assert da.lib.da_kv_append(ctypes.byref(p), good + 2, good, good, good, good, None) == da.DA_ERR_INVALID_ARG
    assert da.lib.da_gqa_decode_attn(ctypes.byref(p), good, good, good, good, None, 0, None) == \
        da.DA_ERR_INVALID_ARG
    assert da.lib.da_gqa_decode_attn(ctypes.byref(p), good, good, good, good, good, 16, None) == \
        da.DA_ERR_WORKSPACE
    assert da.lib.da_gqa_decode_attn_combine(ctypes.byref(p), good, 16, good, good, None) == \
        da.DA_ERR_WORKSPACE
    assert da.lib.da_gqa_decode_attn_combine(ctypes.byref(p), good, 1 << 30, good, good + 8, None) == \
        da.DA_ERR_INVALID_ARG
    bad = P(head_dim=64)
    assert da.lib.da_kv_append(ctypes.byref(bad), good, good, good, good, good, None) == da.DA_ERR_UNSUPPORTED
    assert da.lib.da_kv_append(None, good, good, good, good, good, None) == da.DA_ERR_INVALID_ARG


def test_decode_step_rejects_before_launch():
    p = P()
    buf = (ctypes.c_uint8 * 64)()
    good = ctypes.addressof(buf) + (-ctypes.addressof(buf)) % 16
    args = [good] * 6
    assert da.lib.da_decode_step(ctypes.byref(p), *args, good, 16, good, None) == da.DA_ERR_WORKSPACE
    assert da.lib.da_decode_step(ctypes.byref(p), *args, good, 1 << 30, good + 4, None) == da.DA_ERR_INVALID_ARG
    assert da.lib.da_decode_step(ctypes.byref(p), None, *args[1:], good, 1 << 30, good, None) == \
        da.DA_ERR_INVALID_ARG
    assert da.lib.da_decode_step(ctypes.byref(P(head_dim=64)), *args, good, 1 << 30, good, None) == \
        da.DA_ERR_UNSUPPORTED
    assert da.lib.da_workspace_init(ctypes.byref(p), good, 16, None) == da.DA_ERR_WORKSPACE
    assert da.lib.da_workspace_init(ctypes.byref(p), None, 1 << 30, None) == da.DA_ERR_INVALID_ARG


def test_static_step_rejects_before_launch():
    """da_decode_step_static: bad arguments, and problems whose partials do not fit
    its scratch, return a status before any HIP call (no GPU is needed here)."""
    buf = (ctypes.c_uint8 * 64)()
    good = ctypes.addressof(buf) + (-ctypes.addressof(buf)) % 16
    args = [good] * 6
    p = P()
    assert da.lib.da_decode_step_static(ctypes.byref(p), None, *args[1:], good, None) == da.DA_ERR_INVALID_ARG
    assert da.lib.da_decode_step_static(ctypes.byref(p), *args, good + 4, None) == da.DA_ERR_INVALID_ARG
    assert da.lib.da_decode_step_static(ctypes.byref(P(head_dim=64)), *args, good, None) == da.DA_ERR_UNSUPPORTED
    # fused merge: 1024 heads x 16 slots x 8 rows x 130 floats = 65 MiB > 63 MiB of partials
    big = P(batch=128, n_q_heads=64, n_kv_heads=8, max_seq=65536, merge="launch")
    assert da.plan_attention(big)["fused_combine"]
    assert da.lib.da_decode_step_static(ctypes.byref(big), *args, good, None) == da.DA_ERR_SCRATCH_LIMIT
    # without the fused merge the whole separate-call workspace is needed
    unfused = P(batch=16, q_len=4, n_q_heads=32, n_kv_heads=4, max_seq=8192)  # 65 MiB
    assert not da.plan_attention(unfused)["fused_combine"]
    assert da.lib.da_decode_step_static(ctypes.byref(unfused), *args, good, None) == da.DA_ERR_SCRATCH_LIMIT
    # partials that fit, but more than 8192 (sequence, KV head) arrival counters of 128 bytes
    many = P(batch=1024, n_q_heads=16, n_kv_heads=16, max_seq=128)
    assert da.plan_attention(many)["fused_combine"]
    assert da.lib.da_decode_step_static(ctypes.byref(many), *args, good, None) == da.DA_ERR_SCRATCH_LIMIT
    assert "scratch" in da.status_str(da.DA_ERR_SCRATCH_LIMIT)


@pytest.mark.parametrize("shape,fused", [
    (dict(batch=32, n_q_heads=16, n_kv_heads=8, max_seq=8192), True),    # vector ALU, 2 rows
    (dict(batch=1, n_q_heads=16, n_kv_heads=16, max_seq=4096, dtype="fp16"), True),  # MHA
    (dict(batch=1, max_seq=512), True),
    (dict(batch=1, n_q_heads=16, n_kv_heads=1, max_seq=65536, variant="valu"), False),
    # MFMA: automatic only with at least 128 (sequence, KV head) pairs
    (dict(batch=4, n_q_heads=64, n_kv_heads=8, max_seq=16384), False),   # 32 heads
    (dict(batch=16, n_q_heads=64, n_kv_heads=8, max_seq=1024), True),    # 128 heads
    (dict(batch=16, n_q_heads=16, n_kv_heads=2, head_dim=256, max_seq=8192, dtype="fp16"), False),
    (dict(batch=64, n_q_heads=16, n_kv_heads=2, head_dim=256, max_seq=8192, dtype="fp16"), True),
    (dict(batch=32, q_len=4, n_q_heads=32, n_kv_heads=4, max_seq=8192), False),  # 32 rows x 16 chunks
    # forced into the launch: up to 256 chunk-rows per (sequence, KV head)
    (dict(batch=4, n_q_heads=64, n_kv_heads=8, max_seq=16384, merge="launch"), True),  # 8 rows x 16
    (dict(batch=8, q_len=4, n_q_heads=32, n_kv_heads=4, max_seq=8192, merge="launch"), False),  # 32 rows
    (dict(batch=1, n_q_heads=64, n_kv_heads=8, max_seq=512, merge="launch"), True),   # 8 chunks at most
    (dict(batch=1, n_q_heads=64, n_kv_heads=2, max_seq=65536, merge="launch"), False),  # 32 rows x 16
    (dict(batch=4, q_len=2, n_q_heads=16, n_kv_heads=2, head_dim=256, max_seq=8192, merge="launch"), True),
    (dict(batch=4, q_len=4, n_q_heads=16, n_kv_heads=2, head_dim=256, max_seq=8192, merge="launch"), False),
    # forced out of the launch
    (dict(batch=32, n_q_heads=16, n_kv_heads=8, max_seq=8192, merge="separate"), False),
    (dict(batch=16, n_q_heads=64, n_kv_heads=8, max_seq=1024, merge="separate"), False),
])
def test_plan_fused_merge(shape, fused):
    """The one-launch step merges inside the attention launch when it is allowed to
    (automatically: the vector-ALU kernel, or the MFMA kernels with at least 128
    (sequence, KV head) pairs) and every (sequence, KV head) has few chunk-rows,
    whatever the seq_pos values."""
    pl = da.plan_attention(P(**shape))
    assert pl["fused_combine"] == fused
    units = shape["batch"] * shape.get("n_kv_heads", 8)
    # the counters, one 128-byte line each, sit after the partials
    rows = pl["rows"]
    D = shape.get("head_dim", 128)
    assert pl["workspace_bytes"] >= units * pl["n_chunks"] * rows * (D + 2) * 4 + units * 128


def test_plan_head_dim_256():
    """head_dim 256 always takes the MFMA kernel, one 4-wave workgroup per chunk, aiming
    at 256 chunks like the head_dim-128 MFMA kernel."""
    assert da.plan_attention(P(n_q_heads=64))["target_items"] == 256
    for rows in (1, 8, 32):
        pl = da.plan_attention(P(head_dim=256, n_q_heads=2 * rows, n_kv_heads=2, batch=16))
        assert pl["variant"] == "mfma" and pl["target_items"] == 256
    assert da.workspace_bytes(P(head_dim=256, variant="valu")) == 0


def test_rope_table_must_be_aligned():
    p = P()
    p.rope_freqs = 0x1004  # never dereferenced: rejected before any launch
    assert da.lib.da_plan_attention(ctypes.byref(p), ctypes.byref(da.Plan())) == da.DA_ERR_INVALID_ARG
    p.rope_freqs = 0x1000
    assert da.lib.da_plan_attention(ctypes.byref(p), ctypes.byref(da.Plan())) == da.DA_OK
    p16 = P(n_q_heads=32, n_kv_heads=2, q_len=1, variant="valu")
    p16.rope_freqs = 0x1000
    assert da.lib.da_plan_attention(ctypes.byref(p16), ctypes.byref(da.Plan())) == da.DA_ERR_UNSUPPORTED


def test_paged_problem_checks():
    p = P(max_seq=160)
    pl = da.Plan()
    p.page_size, p.pages_per_seq, p.n_pages, p.block_table = 16, 10, 50, 0x1000
    assert da.lib.da_plan_attention(ctypes.byref(p), ctypes.byref(pl)) == da.DA_OK
    p.block_table = 0x1002  # misaligned
    assert da.lib.da_plan_attention(ctypes.byref(p), ctypes.byref(pl)) == da.DA_ERR_INVALID_ARG
    p.block_table = None
    assert da.lib.da_plan_attention(ctypes.byref(p), ctypes.byref(pl)) == da.DA_ERR_INVALID_ARG
    p.block_table, p.pages_per_seq = 0x1000, 9  # max_seq != pages_per_seq * 16
    assert da.lib.da_plan_attention(ctypes.byref(p), ctypes.byref(pl)) == da.DA_ERR_INVALID_ARG
    p.pages_per_seq, p.page_size, p.max_seq = 5, 32, 160
    assert da.lib.da_plan_attention(ctypes.byref(p), ctypes.byref(pl)) == da.DA_ERR_UNSUPPORTED


def test_status_strings():
    for s in (0, -1, -2, -3, -4):
        assert da.status_str(s) and da.status_str(s) != "unknown status"
    assert da.status_str(5) == "unknown status"


def test_binding_rejects_cpu_tensors():
    import torch
    p = P()
    t = torch.zeros(2, 8, 1024, 128, dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        da.kv_append(p, t, t, t, t, torch.zeros(2, dtype=torch.int32))
