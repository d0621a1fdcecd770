"""CPU oracle for the DSA sparse absorbed-MLA attention path.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke()``
and by the CPU-baseline leg of ``bench.py``; never by the product package.

The arithmetic lives in ``oracle.c`` (plain C, FP64 for attention, fp32 where a
device must reproduce bytes bit for bit).  This module only builds that file
with gcc and marshals numpy arrays into it.  See ``oracle.c`` for the passages
of the SGLang pages each function follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from ctypes import c_double, c_float, c_int, c_int64, c_uint8, c_void_p

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

RAW, SCALED, ROPE, BF16 = 0, 1, 2, 3
ROW_BYTES = {RAW: 512, SCALED: 528, ROPE: 656, BF16: 1024}
ROPE_DIM = 64


def build(src: str = SRC, out: str = LIB, extra_flags: tuple = ()) -> str:
    """Compile ``src`` into a shared library with plain gcc -O2 (no fast-math)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
           "-Wall", "-Werror", *extra_flags, src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def _ptr(a):
    return None if a is None else c_void_p(a.ctypes.data)


def _c(a, dtype):
    if a is None:
        return None
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


class Oracle:
    """ctypes view of one compiled oracle library."""

    def __init__(self, path: str = LIB):
        if not os.path.exists(path) or (
                path == LIB and os.path.getmtime(path) < os.path.getmtime(SRC)):
            build(out=path)
        self.path = path
        lib = ctypes.CDLL(path)
        lib.orc_fp8_decode.restype = c_double
        lib.orc_fp8_decode.argtypes = [c_uint8]
        lib.orc_fp8_encode.restype = c_uint8
        lib.orc_fp8_encode.argtypes = [c_float]
        lib.orc_fp8_encode_array.restype = None
        lib.orc_fp8_encode_array.argtypes = [c_void_p, c_int64, c_void_p]
        lib.orc_fp8_decode_array.restype = None
        lib.orc_fp8_decode_array.argtypes = [c_void_p, c_int64, c_void_p]
        lib.orc_kv_write.restype = c_int64
        lib.orc_kv_write.argtypes = [c_void_p, c_int64, c_int64, c_void_p,
                                     c_void_p, c_int64, c_int]
        lib.orc_q_scale.restype = c_float
        lib.orc_q_scale.argtypes = [c_void_p, c_int64]
        lib.orc_q_quantize.restype = None
        lib.orc_q_quantize.argtypes = [c_void_p, c_int64, c_float, c_void_p]
        lib.orc_resolve.restype = c_int64
        lib.orc_resolve.argtypes = [c_void_p, c_int, c_int, c_void_p, c_void_p,
                                    c_int, c_int, c_void_p, c_int64, c_void_p]
        lib.orc_sparse_attn.restype = c_int64
        lib.orc_topk_transform.argtypes = [c_void_p, c_int, c_int, c_void_p, c_void_p,
                                           c_int, c_int, c_void_p, c_int64, c_int,
                                           c_void_p, c_void_p]
        lib.orc_topk_transform.restype = c_int64
        lib.orc_sparse_attn.argtypes = [
            c_void_p, c_int, c_float, c_int, c_int, c_void_p, c_int64, c_int,
            c_void_p, c_int, c_void_p, c_int, c_int, c_void_p, c_void_p,
            c_float, c_void_p, c_void_p, c_int]
        self.lib = lib

    # -- FP8 codec -----------------------------------------------------------
    def fp8_decode(self, b) -> np.ndarray:
        b = _c(b, np.uint8)
        out = np.empty(b.shape, np.float64)
        self.lib.orc_fp8_decode_array(_ptr(b), b.size, _ptr(out))
        return out

    def fp8_encode(self, x) -> np.ndarray:
        x = _c(x, np.float32)
        out = np.empty(x.shape, np.uint8)
        self.lib.orc_fp8_encode_array(_ptr(x), x.size, _ptr(out))
        return out

    # -- writer --------------------------------------------------------------
    def kv_write(self, kv_bf16, slot_mapping, pool, layout: int) -> int:
        """Write rows of ``kv_bf16`` (uint16 bf16 bits, [n, >=512], or
        [n, >=576] for 656-byte rows) into ``pool`` (uint8 [num_slots,
        row_bytes], modified in place).  Returns errors."""
        kv = np.asarray(kv_bf16)
        assert kv.dtype == np.uint16 and kv.ndim == 2
        assert kv.shape[1] >= 512 + (ROPE_DIM if layout == ROPE else 0)
        assert kv.strides[1] == 2
        sm = _c(slot_mapping, np.int64)
        assert pool.dtype == np.uint8 and pool.flags.c_contiguous
        assert pool.shape[1] == ROW_BYTES[layout]
        return self.lib.orc_kv_write(c_void_p(kv.ctypes.data), kv.shape[0],
                                     kv.strides[0] // 2, _ptr(sm), _ptr(pool),
                                     pool.shape[0], layout)

    # -- query quantisation --------------------------------------------------
    def q_scale(self, q_bf16) -> np.float32:
        q = _c(q_bf16, np.uint16)
        return np.float32(self.lib.orc_q_scale(_ptr(q), q.size))

    def q_quantize(self, q_bf16, scale) -> np.ndarray:
        q = _c(q_bf16, np.uint16)
        out = np.empty(q.shape, np.uint8)
        self.lib.orc_q_quantize(_ptr(q), q.size, c_float(scale), _ptr(out))
        return out

    # -- index resolution ----------------------------------------------------
    def resolve(self, topk, num_slots, page_table=None, page_size=1,
                token_seq=None, seq_lens=None):
        topk = _c(topk, np.int32)
        T, K = topk.shape
        pt = _c(page_table, np.int32)
        max_pages = 0 if pt is None else pt.shape[1]
        slots = np.empty((T, K), np.int64)
        err = self.lib.orc_resolve(_ptr(topk), T, K,
                                   _ptr(_c(token_seq, np.int32)), _ptr(pt),
                                   page_size, max_pages,
                                   _ptr(_c(seq_lens, np.int32)), num_slots,
                                   _ptr(slots))
        return slots, int(err)

    def topk_transform(self, topk, num_slots, k_out, page_table=None, page_size=1,
                       token_seq=None, seq_lens=None):
        """Resolved, compacted rows: (slots int32 [T, k_out], counts int32 [T],
        masked-entry count)."""
        topk = _c(topk, np.int32)
        T, K = topk.shape
        pt = _c(page_table, np.int32)
        max_pages = 0 if pt is None else pt.shape[1]
        out = np.empty((T, k_out), np.int32)
        counts = np.empty(T, np.int32)
        err = self.lib.orc_topk_transform(_ptr(topk), T, K,
                                          _ptr(_c(token_seq, np.int32)), _ptr(pt),
                                          page_size, max_pages,
                                          _ptr(_c(seq_lens, np.int32)), num_slots,
                                          k_out, _ptr(out), _ptr(counts))
        return out, counts, int(err)

    # -- attention -----------------------------------------------------------
    def sparse_attn(self, q, pool, layout, topk, softmax_scale, *,
                    q_scale=None, page_table=None, page_size=1,
                    token_seq=None, seq_lens=None, nthreads=None):
        """Returns (out f64 [T,H,512], lse f64 [T,H], err_count).

        ``q`` is uint16 bf16 bits [T,H,512] ([T,H,576] for 656-byte rows:
        latent then RoPE part), or uint8 FP8 codes when ``q_scale`` is
        given."""
        is_fp8 = q_scale is not None
        q = _c(q, np.uint8 if is_fp8 else np.uint16)
        T, H, Dq = q.shape
        D = 512
        assert Dq == D + (ROPE_DIM if layout == ROPE else 0)
        topk = _c(topk, np.int32)
        assert topk.shape[0] == T
        K = topk.shape[1]
        assert pool.dtype == np.uint8 and pool.shape[1] == ROW_BYTES[layout]
        pool = np.ascontiguousarray(pool)
        pt = _c(page_table, np.int32)
        max_pages = 0 if pt is None else pt.shape[1]
        out = np.empty((T, H, D), np.float64)
        lse = np.empty((T, H), np.float64)
        if nthreads is None:
            nthreads = os.cpu_count() or 1
        err = self.lib.orc_sparse_attn(
            _ptr(q), int(is_fp8), c_float(q_scale if is_fp8 else 1.0), T, H,
            _ptr(pool), pool.shape[0], layout, _ptr(topk), K, _ptr(pt),
            page_size, max_pages, _ptr(_c(token_seq, np.int32)),
            _ptr(_c(seq_lens, np.int32)), c_float(softmax_scale), _ptr(out),
            _ptr(lse), int(nthreads))
        return out, lse, int(err)


_default = None


def get() -> Oracle:
    """The oracle built from ``oracle.c`` (compiled on first use)."""
    global _default
    if _default is None:
        _default = Oracle(LIB)
    return _default
