"""MI355X-native decode attention with KV-cache append.

Thin ctypes binding over the C ABI in ``include/decode_attn.h`` (library
``libdecode_attn.so``, built by ``build_lib.py``).  The functions here only
marshal arguments: check that tensors are on the GPU, contiguous and of the
declared shape and type, then pass raw device pointers and the current HIP
stream.  Every step of the computation runs in the library's HIP kernels;
there is no fallback of any kind, and importing the binding fails loudly if
the library has not been built.

Names follow the C entry points without their ``da_`` prefix:
``kv_append``, ``gqa_decode_attn``, ``gqa_decode_attn_combine``,
``decode_step`` (the one-launch step), ``decode_step_static`` (the same without
a workspace), ``workspace_init``,
``workspace_bytes``, ``plan_attention``.  ``decode_step_separate`` runs the
three separate calls in order.
"""
import ctypes
import os

import torch

from . import workloads  # noqa: F401  (seeded input generator, no method arithmetic)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdecode_attn.so")

DA_OK, DA_ERR_INVALID_ARG, DA_ERR_UNSUPPORTED, DA_ERR_WORKSPACE, DA_ERR_HIP = 0, -1, -2, -3, -4
DA_ERR_SCRATCH_LIMIT = -5
DA_BF16, DA_FP16 = 0, 1
VARIANTS = {0: "valu", 1: "mfma"}
_DTYPE_CODE = {torch.bfloat16: DA_BF16, torch.float16: DA_FP16}


class DecodeAttnError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_str(status)} (status {status})")
        self.status = status


class Problem(ctypes.Structure):
    """Mirror of ``da_problem``."""
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("q_len", ctypes.c_int32),
        ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("max_seq", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("chunk_tokens", ctypes.c_int32),
        ("variant", ctypes.c_int32),
        ("work_items", ctypes.c_int32),
        ("rope_freqs", ctypes.c_void_p),
        ("page_size", ctypes.c_int32),
        ("pages_per_seq", ctypes.c_int32),
        ("n_pages", ctypes.c_int32),
        ("block_table", ctypes.c_void_p),
        ("rope_dim", ctypes.c_int32),
        ("out_gate", ctypes.c_void_p),
        ("merge", ctypes.c_int32),
    ]

    def __repr__(self):
        f = ", ".join(f"{n}={getattr(self, n)}" for n, _ in self._fields_)
        return f"Problem({f})"


class Plan(ctypes.Structure):
    """Mirror of ``da_plan``."""
    _fields_ = [
        ("chunk_tokens", ctypes.c_int32),
        ("n_chunks", ctypes.c_int32),
        ("rows", ctypes.c_int32),
        ("variant", ctypes.c_int32),
        ("balanced", ctypes.c_int32),
        ("target_items", ctypes.c_int32),
        ("items", ctypes.c_int32),
        ("fused_combine", ctypes.c_int32),
        ("workspace_bytes", ctypes.c_size_t),
    ]


EXPORTS = ("da_plan_attention", "da_workspace_bytes", "da_kv_append", "da_gqa_decode_attn",
           "da_gqa_decode_attn_combine", "da_workspace_init", "da_decode_step", "da_decode_step_static",
           "da_chunk_layout", "da_status_str")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with 'python -m decode_attention_append_amd.build_lib' "
            "(the HIP library is required; there is no fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, sz, i32p = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p
    pp = ctypes.POINTER(Problem)
    lib.da_plan_attention.argtypes = [pp, ctypes.POINTER(Plan)]
    lib.da_plan_attention.restype = ctypes.c_int
    lib.da_workspace_bytes.argtypes = [pp]
    lib.da_workspace_bytes.restype = sz
    lib.da_kv_append.argtypes = [pp, vp, vp, vp, vp, i32p, vp]
    lib.da_kv_append.restype = ctypes.c_int
    lib.da_gqa_decode_attn.argtypes = [pp, vp, vp, vp, i32p, vp, sz, vp]
    lib.da_gqa_decode_attn.restype = ctypes.c_int
    lib.da_gqa_decode_attn_combine.argtypes = [pp, vp, sz, i32p, vp, vp]
    lib.da_gqa_decode_attn_combine.restype = ctypes.c_int
    lib.da_workspace_init.argtypes = [pp, vp, sz, vp]
    lib.da_workspace_init.restype = ctypes.c_int
    lib.da_decode_step.argtypes = [pp, vp, vp, vp, vp, vp, i32p, vp, sz, vp, vp]
    lib.da_decode_step.restype = ctypes.c_int
    lib.da_decode_step_static.argtypes = [pp, vp, vp, vp, vp, vp, i32p, vp, vp]
    lib.da_decode_step_static.restype = ctypes.c_int
    lib.da_chunk_layout.argtypes = [pp, vp, vp, vp]
    lib.da_chunk_layout.restype = ctypes.c_int
    lib.da_status_str.argtypes = [ctypes.c_int]
    lib.da_status_str.restype = ctypes.c_char_p
    return lib


_lib = None


def _get_lib():
    global _lib
    if _lib is None:
        _lib = _load()
    return _lib


def __getattr__(name):
    # ``lib`` (the ctypes handle) loads on first use, so that building the library
    # does not need an already-built one; a missing library still fails loudly there.
    if name == "lib":
        return _get_lib()
    raise AttributeError(name)


def status_str(status: int) -> str:
    return _get_lib().da_status_str(status).decode()


def problem(batch, q_len, n_q_heads, n_kv_heads, head_dim, max_seq, dtype, scale=0.0,
            chunk_tokens=0, variant=None, work_items=0, rope_freqs=None, block_table=None,
            n_pages=0, page_size=16, rope_dim=0, out_gate=None, merge=None) -> Problem:
    """variant: None (automatic), "valu" or "mfma"; chunk_tokens 0 = balanced chunks.
    rope_freqs: None, or a float32 GPU tensor of head_dim/2 rotary frequencies.
    block_table: None (contiguous caches), or an int32 GPU tensor [batch, pages_per_seq]
    for paged caches (pools [n_pages, n_kv_heads, page_size, head_dim]; max_seq must be
    pages_per_seq * page_size).  rope_dim: rotate only the first rope_dim dims (0: all;
    rope_freqs then holds rope_dim/2 values).  out_gate: None, or a GPU tensor
    [batch, q_len, n_q_heads, head_dim] of the element type: the output is multiplied
    by sigmoid(out_gate).  merge: None (automatic), "launch" (da_decode_step merges inside
    the attention launch whenever the plan allows it) or "separate" (always the combine
    launch).  The problem keeps references to the tensors."""
    if isinstance(dtype, torch.dtype):
        dtype = _DTYPE_CODE[dtype]
    elif isinstance(dtype, str):
        dtype = {"bf16": DA_BF16, "fp16": DA_FP16}[dtype]
    v = 0 if variant is None else {"valu": 1, "mfma": 2}[variant]
    rp = None
    if rope_freqs is not None:
        rp = _dev(rope_freqs, "rope_freqs", ((rope_dim or head_dim) // 2,), torch.float32)
    og = None
    if out_gate is not None:
        og = _dev(out_gate, "out_gate", (batch, q_len, n_q_heads, head_dim),
                  {DA_BF16: torch.bfloat16, DA_FP16: torch.float16}[dtype])
    ps, pps, bt = 0, 0, None
    if block_table is not None:
        if block_table.dim() != 2 or block_table.shape[0] != batch:
            raise ValueError("block_table must be [batch, pages_per_seq]")
        pps = block_table.shape[1]
        bt = _dev(block_table, "block_table", None, torch.int32)
        ps = page_size
    mg = {None: 0, "launch": 1, "separate": 2}[merge]
    pr = Problem(batch, q_len, n_q_heads, n_kv_heads, head_dim, max_seq, dtype, float(scale),
                 chunk_tokens, v, work_items, rp, ps, pps, n_pages if ps else 0, bt, rope_dim, og, mg)
    pr._refs = (rope_freqs, block_table, out_gate)  # keeps the tensors alive as long as the problem
    return pr


def problem_for(q: torch.Tensor, k_cache: torch.Tensor, scale=0.0, chunk_tokens=0,
                variant=None, work_items=0, rope_freqs=None, block_table=None, rope_dim=0,
                out_gate=None, merge=None) -> Problem:
    """The problem described by q [B, q_len, Hq, D] and a cache [B, Hkv, S, D], or with a
    block table [B, pages_per_seq] a page pool [n_pages, Hkv, page_size, D]."""
    B, q_len, Hq, D = q.shape
    if block_table is None:
        _, Hkv, S, _ = k_cache.shape
        return problem(B, q_len, Hq, Hkv, D, S, q.dtype, scale, chunk_tokens, variant, work_items, rope_freqs,
                       rope_dim=rope_dim, out_gate=out_gate, merge=merge)
    n_pages, Hkv, page_size, _ = k_cache.shape
    S = block_table.shape[1] * page_size
    return problem(B, q_len, Hq, Hkv, D, S, q.dtype, scale, chunk_tokens, variant, work_items, rope_freqs,
                   block_table, n_pages, page_size, rope_dim, out_gate, merge)


def plan_attention(p: Problem) -> dict:
    pl = Plan()
    st = _get_lib().da_plan_attention(ctypes.byref(p), ctypes.byref(pl))
    if st != DA_OK:
        raise DecodeAttnError(st, "da_plan_attention")
    return {"chunk_tokens": pl.chunk_tokens, "n_chunks": pl.n_chunks, "rows": pl.rows,
            "variant": VARIANTS[pl.variant], "balanced": bool(pl.balanced),
            "target_items": pl.target_items, "items": pl.items,
            "fused_combine": bool(pl.fused_combine), "workspace_bytes": pl.workspace_bytes}


def chunk_layout(p: Problem, seq_pos) -> list:
    """[(n_chunks, chunk_len)] per sequence for these seq_pos values (host computation)."""
    import numpy as np
    sp = np.ascontiguousarray(np.asarray(seq_pos, dtype=np.int32))
    if sp.shape != (p.batch,):
        raise ValueError("seq_pos must have one value per sequence")
    n = np.zeros(p.batch, dtype=np.int32)
    ln = np.zeros(p.batch, dtype=np.int32)
    st = _get_lib().da_chunk_layout(ctypes.byref(p), sp.ctypes.data, n.ctypes.data, ln.ctypes.data)
    if st != DA_OK:
        raise DecodeAttnError(st, "da_chunk_layout")
    return list(zip(n.tolist(), ln.tolist()))


def workspace_bytes(p: Problem) -> int:
    return _get_lib().da_workspace_bytes(ctypes.byref(p))


def new_workspace(p: Problem, device="cuda", stream=None) -> torch.Tensor:
    """A uint8 device buffer of workspace_bytes(p) (allocated by torch, owned by the
    caller), prepared by workspace_init on ``stream``."""
    n = workspace_bytes(p)
    if n == 0:
        raise DecodeAttnError(DA_ERR_INVALID_ARG, "workspace_bytes")
    ws = torch.empty(n, dtype=torch.uint8, device=device)
    workspace_init(p, ws, stream)
    return ws


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _dev(t: torch.Tensor, name: str, shape=None, dtype=None) -> ctypes.c_void_p:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    return ctypes.c_void_p(t.data_ptr())


def _elem(p: Problem):
    return torch.float16 if p.dtype == DA_FP16 else torch.bfloat16


def _cache_shape(p: Problem):
    if p.page_size:
        return (p.n_pages, p.n_kv_heads, p.page_size, p.head_dim)
    return (p.batch, p.n_kv_heads, p.max_seq, p.head_dim)


def kv_append(p: Problem, k_cache, v_cache, k_new, v_new, seq_pos, stream=None):
    """da_kv_append: k_cache[b, h, seq_pos[b] + i] = k_new[b, i, h] (and V), in place."""
    e = _elem(p)
    cs = _cache_shape(p)
    ns = (p.batch, p.q_len, p.n_kv_heads, p.head_dim)
    st = _get_lib().da_kv_append(ctypes.byref(p), _dev(k_cache, "k_cache", cs, e), _dev(v_cache, "v_cache", cs, e),
                          _dev(k_new, "k_new", ns, e), _dev(v_new, "v_new", ns, e),
                          _dev(seq_pos, "seq_pos", (p.batch,), torch.int32), _stream(stream))
    if st != DA_OK:
        raise DecodeAttnError(st, "da_kv_append")


def gqa_decode_attn(p: Problem, q, k_cache, v_cache, seq_pos, workspace, stream=None):
    """da_gqa_decode_attn: fp32 split-context partials into ``workspace``."""
    e = _elem(p)
    cs = _cache_shape(p)
    st = _get_lib().da_gqa_decode_attn(ctypes.byref(p),
                                _dev(q, "q", (p.batch, p.q_len, p.n_q_heads, p.head_dim), e),
                                _dev(k_cache, "k_cache", cs, e), _dev(v_cache, "v_cache", cs, e),
                                _dev(seq_pos, "seq_pos", (p.batch,), torch.int32),
                                _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
                                _stream(stream))
    if st != DA_OK:
        raise DecodeAttnError(st, "da_gqa_decode_attn")


def gqa_decode_attn_combine(p: Problem, workspace, seq_pos, out, stream=None):
    """da_gqa_decode_attn_combine: merge the partials into ``out`` [B, q_len, Hq, D]."""
    e = _elem(p)
    st = _get_lib().da_gqa_decode_attn_combine(
        ctypes.byref(p), _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _dev(seq_pos, "seq_pos", (p.batch,), torch.int32),
        _dev(out, "out", (p.batch, p.q_len, p.n_q_heads, p.head_dim), e), _stream(stream))
    if st != DA_OK:
        raise DecodeAttnError(st, "da_gqa_decode_attn_combine")


def workspace_init(p: Problem, workspace, stream=None):
    """da_workspace_init: zero the one-launch step's arrival counters in ``workspace``."""
    st = _get_lib().da_workspace_init(ctypes.byref(p), _dev(workspace, "workspace"),
                                      workspace.numel() * workspace.element_size(), _stream(stream))
    if st != DA_OK:
        raise DecodeAttnError(st, "da_workspace_init")


def decode_step(p: Problem, q, k_cache, v_cache, k_new, v_new, seq_pos, workspace, out, stream=None):
    """da_decode_step: append + attention + combine, in one launch where the plan allows."""
    e = _elem(p)
    cs = _cache_shape(p)
    ns = (p.batch, p.q_len, p.n_kv_heads, p.head_dim)
    qs = (p.batch, p.q_len, p.n_q_heads, p.head_dim)
    st = _get_lib().da_decode_step(
        ctypes.byref(p), _dev(q, "q", qs, e), _dev(k_cache, "k_cache", cs, e), _dev(v_cache, "v_cache", cs, e),
        _dev(k_new, "k_new", ns, e), _dev(v_new, "v_new", ns, e),
        _dev(seq_pos, "seq_pos", (p.batch,), torch.int32),
        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _dev(out, "out", qs, e), _stream(stream))
    if st != DA_OK:
        raise DecodeAttnError(st, "da_decode_step")


def decode_step_static(p: Problem, q, k_cache, v_cache, k_new, v_new, seq_pos, out, stream=None):
    """da_decode_step_static: da_decode_step with the library's own scratch instead of a
    workspace (nothing is allocated; calls on one GPU must not overlap)."""
    e = _elem(p)
    cs = _cache_shape(p)
    ns = (p.batch, p.q_len, p.n_kv_heads, p.head_dim)
    qs = (p.batch, p.q_len, p.n_q_heads, p.head_dim)
    st = _get_lib().da_decode_step_static(
        ctypes.byref(p), _dev(q, "q", qs, e), _dev(k_cache, "k_cache", cs, e), _dev(v_cache, "v_cache", cs, e),
        _dev(k_new, "k_new", ns, e), _dev(v_new, "v_new", ns, e),
        _dev(seq_pos, "seq_pos", (p.batch,), torch.int32), _dev(out, "out", qs, e), _stream(stream))
    if st != DA_OK:
        raise DecodeAttnError(st, "da_decode_step_static")


def decode_step_separate(p: Problem, q, k_cache, v_cache, k_new, v_new, seq_pos, workspace, out,
                         stream=None):
    """The three separate calls of one decode step, in order, on one stream."""
    kv_append(p, k_cache, v_cache, k_new, v_new, seq_pos, stream)
    gqa_decode_attn(p, q, k_cache, v_cache, seq_pos, workspace, stream)
    gqa_decode_attn_combine(p, workspace, seq_pos, out, stream)
