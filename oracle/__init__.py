"""Reference oracle for the decode-attention step (TEST INFRASTRUCTURE ONLY).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never uses it.

Python side of ``oracle.c``: argument marshalling with ctypes and numpy, no
arithmetic of the method.  ``oracle.c`` says what is computed and which
passages of the pages each step follows.
"""
import ctypes
import os

import numpy as np

from . import build_oracle

BF16 = 0
FP16 = 1


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _u16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        if a.dtype.itemsize != 2:
            raise TypeError(f"expected 16-bit element patterns, got {a.dtype}")
        a = a.view(np.uint16)
    return a


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


class Oracle:
    """The oracle library at ``path`` (default: the built ``liboracle.so``)."""

    def __init__(self, path: str = None):
        if path is None:
            path = build_oracle.LIB
            if not os.path.exists(path):
                build_oracle.build()
        lib = ctypes.CDLL(path)
        i32, f64, p = ctypes.c_int32, ctypes.c_double, ctypes.c_void_p
        lib.oracle_decode_bf16.argtypes = [ctypes.c_uint16]
        lib.oracle_decode_bf16.restype = f64
        lib.oracle_decode_fp16.argtypes = [ctypes.c_uint16]
        lib.oracle_decode_fp16.restype = f64
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_kv_append.argtypes = [i32] * 5 + [p] * 5
        lib.oracle_kv_append.restype = ctypes.c_int
        lib.oracle_attend_row.argtypes = [i32] * 5 + [f64] + [p] * 5
        lib.oracle_attend_row.restype = i32
        lib.oracle_gqa_decode.argtypes = [i32] * 7 + [f64] + [p] * 6
        lib.oracle_gqa_decode.restype = ctypes.c_int
        lib.oracle_gqa_decode_rows.argtypes = [i32] * 7 + [f64] + [p] * 4 + [i32] + [p] * 4
        lib.oracle_gqa_decode_rows.restype = ctypes.c_int
        lib.oracle_encode_bf16.argtypes = [f64]
        lib.oracle_encode_bf16.restype = ctypes.c_uint16
        lib.oracle_encode_fp16.argtypes = [f64]
        lib.oracle_encode_fp16.restype = ctypes.c_uint16
        lib.oracle_rope_rows.argtypes = [i32, i32, i32, i32, p, p, p, p]
        lib.oracle_rope_rows.restype = ctypes.c_int
        lib.oracle_output_gate.argtypes = [i32, ctypes.c_int64, p, p]
        lib.oracle_output_gate.restype = None
        lib.oracle_gather_paged.argtypes = [i32] * 6 + [p] * 3
        lib.oracle_gather_paged.restype = ctypes.c_int
        lib.oracle_kv_append_paged.argtypes = [i32] * 7 + [p] * 6
        lib.oracle_kv_append_paged.restype = ctypes.c_int
        self.lib = lib
        self.path = path

    def num_threads(self) -> int:
        return self.lib.oracle_num_threads()

    def decode(self, bits, dtype: int) -> np.ndarray:
        """16-bit patterns -> float64, element by element through the C decoder."""
        f = self.lib.oracle_decode_fp16 if dtype == FP16 else self.lib.oracle_decode_bf16
        bits = _u16(bits)
        flat = bits.ravel()
        return np.array([f(int(x)) for x in flat], dtype=np.float64).reshape(bits.shape)

    def encode(self, values, dtype: int) -> np.ndarray:
        """float64 -> 16-bit patterns (round to nearest even), element by element in C."""
        f = self.lib.oracle_encode_fp16 if dtype == FP16 else self.lib.oracle_encode_bf16
        v = np.asarray(values, dtype=np.float64)
        return np.array([f(float(x)) for x in v.ravel()], dtype=np.uint16).reshape(v.shape)

    def rope_rows(self, rows, positions, freqs, dtype: int) -> np.ndarray:
        """Rotary embedding of ``rows`` [..., D] (16-bit patterns) at ``positions`` (one per
        row, shape rows.shape[:-1]) with the float32 ``freqs``: R/2 values rotate the first
        R dims (R = D for full rotation); returns new patterns."""
        x = _u16(rows)
        D = x.shape[-1]
        pos = _i32(positions).reshape(-1)
        if pos.size * D != x.size:
            raise ValueError("one position per row")
        f = np.ascontiguousarray(np.asarray(freqs, dtype=np.float32).reshape(-1))
        R = 2 * f.size
        out = np.empty_like(x)
        if self.lib.oracle_rope_rows(dtype, pos.size, D, R, _ptr(pos), _ptr(f), _ptr(x), _ptr(out)) != 0:
            raise ValueError("bad row length or rotary width")
        return out

    def output_gate(self, out, gate, dtype: int) -> np.ndarray:
        """out (float64 attention output) times sigmoid(gate) elementwise; gate: 16-bit
        patterns of the same shape.  Returns a new array."""
        o = np.ascontiguousarray(np.array(out, dtype=np.float64))
        g = _u16(gate)
        if g.shape != o.shape:
            raise ValueError("gate and output shapes differ")
        self.lib.oracle_output_gate(dtype, o.size, _ptr(g), _ptr(o))
        return o

    def rope_q(self, q, seq_pos, freqs, dtype: int) -> np.ndarray:
        """q [B, q_len, Hq, D] rotated at position seq_pos[b] + i (new patterns)."""
        q = _u16(q)
        B, q_len, Hq, _ = q.shape
        pos = _i32(seq_pos)[:, None, None] + np.arange(q_len, dtype=np.int32)[None, :, None]
        return self.rope_rows(q, np.broadcast_to(pos, (B, q_len, Hq)), freqs, dtype)

    def kv_append_rope(self, k_cache, v_cache, k_new, v_new, seq_pos, freqs, dtype: int):
        """The append with the new K rows rotated at their positions seq_pos[b] + i first
        (V rows unchanged); returns (k_cache', v_cache')."""
        kn = _u16(k_new)
        B, q_len, Hkv, _ = kn.shape
        pos = _i32(seq_pos)[:, None, None] + np.arange(q_len, dtype=np.int32)[None, :, None]
        k_rot = self.rope_rows(kn, np.broadcast_to(pos, (B, q_len, Hkv)), freqs, dtype)
        return self.kv_append(k_cache, v_cache, k_rot, v_new, seq_pos)

    def gather_paged(self, pool, block_table):
        """Page pool [n_pages, Hkv, page_size, D] + block table [B, pages_per_seq] -> the
        sequences' contiguous caches [B, Hkv, pages_per_seq * page_size, D]."""
        pool = _u16(pool)
        n_pages, Hkv, page_size, D = pool.shape
        bt = _i32(block_table)
        B, pps = bt.shape
        out = np.empty((B, Hkv, pps * page_size, D), dtype=np.uint16)
        if self.lib.oracle_gather_paged(B, Hkv, D, page_size, pps, n_pages, _ptr(bt), _ptr(pool), _ptr(out)):
            raise ValueError("block table entry outside the pool")
        return out

    def kv_append_paged(self, k_pool, v_pool, k_new, v_new, seq_pos, block_table):
        """The append into page pools; returns (k_pool', v_pool') as new arrays."""
        kp, vp = _u16(k_pool).copy(), _u16(v_pool).copy()
        n_pages, Hkv, page_size, D = kp.shape
        kn, vn = _u16(k_new), _u16(v_new)
        B, q_len = kn.shape[:2]
        bt = _i32(block_table)
        sp = _i32(seq_pos)
        if self.lib.oracle_kv_append_paged(B, q_len, Hkv, D, page_size, bt.shape[1], n_pages, _ptr(bt), _ptr(sp),
                                           _ptr(kn), _ptr(vn), _ptr(kp), _ptr(vp)):
            raise ValueError("block table entry outside the pool, or seq_pos outside the pages")
        return kp, vp

    def kv_append(self, k_cache, v_cache, k_new, v_new, seq_pos):
        """Returns (k_cache', v_cache') as new uint16 arrays; the inputs are not modified.

        k_cache/v_cache: [B, Hkv, S, D]; k_new/v_new: [B, q_len, Hkv, D]; seq_pos: [B].
        """
        kc = _u16(k_cache).copy()
        vc = _u16(v_cache).copy()
        kn, vn = _u16(k_new), _u16(v_new)
        B, Hkv, S, D = kc.shape
        q_len = kn.shape[1]
        if kn.shape != (B, q_len, Hkv, D) or vn.shape != kn.shape or vc.shape != kc.shape:
            raise ValueError("shape mismatch")
        sp = _i32(seq_pos)
        rc = self.lib.oracle_kv_append(B, q_len, Hkv, D, S, _ptr(sp), _ptr(kn), _ptr(vn),
                                       _ptr(kc), _ptr(vc))
        if rc != 0:
            raise ValueError("seq_pos out of range for the cache")
        return kc, vc

    def gqa_decode(self, q, k_cache, v_cache, seq_pos, dtype: int, scale: float = None,
                   with_weights: bool = False):
        """Attention of every query row over the (already appended) cache.

        q: [B, q_len, Hq, D]; caches [B, Hkv, S, D]; returns float64 out [B, q_len, Hq, D]
        (and the softmax weights [B, q_len, Hq, S] when asked).
        """
        q, kc, vc = _u16(q), _u16(k_cache), _u16(v_cache)
        B, q_len, Hq, D = q.shape
        _, Hkv, S, _ = kc.shape
        if scale is None:
            scale = 1.0 / np.sqrt(D)
        sp = _i32(seq_pos)
        out = np.empty((B, q_len, Hq, D), dtype=np.float64)
        w = np.empty((B, q_len, Hq, S), dtype=np.float64) if with_weights else None
        rc = self.lib.oracle_gqa_decode(dtype, B, q_len, Hq, Hkv, D, S, float(scale), _ptr(sp),
                                        _ptr(q), _ptr(kc), _ptr(vc), _ptr(out), _ptr(w))
        if rc != 0:
            raise ValueError("bad problem description")
        return (out, w) if with_weights else out

    def gqa_decode_rows(self, q, k_cache, v_cache, seq_pos, rows, dtype: int,
                        scale: float = None):
        """Selected output rows: ``rows`` is [n, 3] of (b, i, hq); returns [n, D] float64."""
        q, kc, vc = _u16(q), _u16(k_cache), _u16(v_cache)
        B, q_len, Hq, D = q.shape
        _, Hkv, S, _ = kc.shape
        if scale is None:
            scale = 1.0 / np.sqrt(D)
        rows = _i32(rows).reshape(-1, 3)
        rb, ri, rh = (np.ascontiguousarray(rows[:, k]) for k in range(3))
        sp = _i32(seq_pos)
        out = np.empty((rows.shape[0], D), dtype=np.float64)
        rc = self.lib.oracle_gqa_decode_rows(dtype, B, q_len, Hq, Hkv, D, S, float(scale),
                                             _ptr(sp), _ptr(q), _ptr(kc), _ptr(vc),
                                             rows.shape[0], _ptr(rb), _ptr(ri), _ptr(rh),
                                             _ptr(out))
        if rc != 0:
            raise ValueError("bad problem description or row index")
        return out


_default = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def num_threads() -> int:
    return default().num_threads()


def decode(bits, dtype):
    return default().decode(bits, dtype)


def kv_append(*args, **kw):
    return default().kv_append(*args, **kw)


def gqa_decode(*args, **kw):
    return default().gqa_decode(*args, **kw)


def gqa_decode_rows(*args, **kw):
    return default().gqa_decode_rows(*args, **kw)


def encode(values, dtype):
    return default().encode(values, dtype)


def rope_rows(*args, **kw):
    return default().rope_rows(*args, **kw)


def rope_q(*args, **kw):
    return default().rope_q(*args, **kw)


def kv_append_rope(*args, **kw):
    return default().kv_append_rope(*args, **kw)


def gather_paged(*args, **kw):
    return default().gather_paged(*args, **kw)


def kv_append_paged(*args, **kw):
    return default().kv_append_paged(*args, **kw)


def output_gate(*args, **kw):
    return default().output_gate(*args, **kw)
