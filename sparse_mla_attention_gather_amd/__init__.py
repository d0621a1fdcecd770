"""Python binding of the gfx950 DSA sparse absorbed-MLA attention library.

Argument marshalling only: every function forwards to the C ABI of
``include/dsa.h`` (same names, same argument order) in the in-tree HIP library
``libdsa_mi355x.so``; every step of the computation runs in its kernels.
Pointer arguments accept a ``torch.Tensor`` (its ``data_ptr()``), an ``int``
address, or ``None``; ``stream=None`` means torch's current stream.  Each call
returns the ``dsa_status`` integer; ``check()`` turns a nonzero one into
``DsaError``.  There is no fallback: importing this package without the built
library raises ``ImportError``.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import c_float, c_int32, c_int64, c_size_t, c_void_p

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdsa_mi355x.so")

# enums of include/dsa.h
DSA_KV_RAW_FP8_512, DSA_KV_SCALED_FP8_528, DSA_KV_SCALED_FP8_656, DSA_KV_BF16_1024 = 0, 1, 2, 3
DSA_BF16, DSA_FP32, DSA_FP8_E4M3FN, DSA_FP8_E4M3FNUZ = 0, 1, 2, 3
STATUS = ["DSA_OK", "DSA_ERR_NULL", "DSA_ERR_SHAPE", "DSA_ERR_WIDTH_MISMATCH",
          "DSA_ERR_LAYOUT", "DSA_ERR_DTYPE", "DSA_ERR_ALIGN",
          "DSA_ERR_WORKSPACE", "DSA_ERR_DEVICE", "DSA_ERR_LAUNCH"]
for _i, _n in enumerate(STATUS):
    globals()[_n] = _i

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with "
        "`python -m sparse_mla_attention_gather_amd.build` (hipcc, gfx950)")

# PyTorch ships its own copy of the HIP runtime.  Loading it first makes this
# library bind to that same runtime instance (one device context, one set of
# streams); loaded the other way round, the process would hold two runtimes
# and the library would not see torch's device state.
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)

_SIGS = {
    "dsa_kv_row_bytes": (c_int32, [c_int32]),
    "dsa_status_string": (ctypes.c_char_p, [c_int32]),
    "dsa_kv_write": (c_int32, [c_void_p, c_int64, c_int64, c_int32, c_int32,
                               c_int32, c_void_p, c_void_p, c_int64, c_int32,
                               c_int32, c_void_p, c_void_p]),
    "dsa_quantize_q_fp8": (c_int32, [c_void_p, c_int64, c_int32, c_void_p,
                                     c_void_p, c_int32, c_int32, c_void_p,
                                     c_size_t, c_void_p]),
    "dsa_quantize_q_workspace_bytes": (c_size_t, [c_int64]),
    "dsa_attn_workspace_bytes": (c_size_t, [c_int32, c_int32, c_int32, c_int32]),
}
_ATTN_ARGS = [c_void_p, c_int32, c_void_p, c_int32, c_int32, c_int32, c_int32,
              c_void_p, c_int64, c_int32, c_int32, c_void_p, c_int32, c_void_p,
              c_int32, c_int32, c_int32, c_void_p, c_void_p, c_float, c_void_p,
              c_int32, c_void_p, c_void_p, c_size_t, c_void_p, c_void_p]
_SIGS["dsa_sparse_attn_decode"] = (c_int32, _ATTN_ARGS)
# the workspace pointer and its size are the 24th and 25th arguments
_SIGS["dsa_sparse_attn_decode_noalloc"] = (c_int32, _ATTN_ARGS[:23] + _ATTN_ARGS[25:])
_SIGS["dsa_sparse_attn_prefill"] = (c_int32, _ATTN_ARGS)
_SIGS["dsa_topk_transform"] = (c_int32, [c_void_p, c_int32, c_int32, c_void_p, c_int32,
                                         c_int32, c_int32, c_void_p, c_void_p, c_int64,
                                         c_void_p, c_int32, c_void_p, c_void_p, c_void_p])
for _name, (_res, _args) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args

EXPORTED = tuple(_SIGS)


class DsaError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        super().__init__(dsa_status_string(status))


def check(status: int) -> None:
    if status != 0:
        raise DsaError(status)


def _p(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _s(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def dsa_kv_row_bytes(layout: int) -> int:
    return _lib.dsa_kv_row_bytes(layout)


def dsa_status_string(status: int) -> str:
    return _lib.dsa_status_string(status).decode()


def dsa_kv_write(kv, n, kv_row_stride, kv_dtype, kv_dim, rope_dim,
                 slot_mapping, pool, num_slots, layout, fp8_format,
                 err_count=None, stream=None) -> int:
    return _lib.dsa_kv_write(_p(kv), n, kv_row_stride, kv_dtype, kv_dim,
                             rope_dim, _p(slot_mapping), _p(pool), num_slots,
                             layout, fp8_format, _p(err_count), _s(stream))


def dsa_quantize_q_fp8(q, n_elems, q_dtype, q8, q_scale, scale_given,
                       fp8_format, workspace=None, workspace_bytes=0,
                       stream=None) -> int:
    return _lib.dsa_quantize_q_fp8(_p(q), n_elems, q_dtype, _p(q8),
                                   _p(q_scale), scale_given, fp8_format,
                                   _p(workspace), workspace_bytes, _s(stream))


def dsa_quantize_q_workspace_bytes(n_elems: int) -> int:
    return _lib.dsa_quantize_q_workspace_bytes(n_elems)


def dsa_attn_workspace_bytes(T: int, H: int, K: int, phase: int) -> int:
    return _lib.dsa_attn_workspace_bytes(T, H, K, phase)


def _attn(fn, q, q_dtype, q_scale, T, H, D, rope_dim, pool, num_slots, layout,
          fp8_format, topk, K, page_table, page_size, max_pages, num_seqs,
          token_seq, seq_lens, softmax_scale, out, out_dtype, lse, workspace,
          workspace_bytes, err_count, stream):
    return fn(_p(q), q_dtype, _p(q_scale), T, H, D, rope_dim, _p(pool),
              num_slots, layout, fp8_format, _p(topk), K, _p(page_table),
              page_size, max_pages, num_seqs, _p(token_seq), _p(seq_lens),
              softmax_scale, _p(out), out_dtype, _p(lse), _p(workspace),
              workspace_bytes, _p(err_count), _s(stream))


def dsa_sparse_attn_decode(q, q_dtype, q_scale, T, H, D, rope_dim, pool,
                           num_slots, layout, fp8_format, topk, K, page_table,
                           page_size, max_pages, num_seqs, token_seq, seq_lens,
                           softmax_scale, out, out_dtype, lse=None,
                           workspace=None, workspace_bytes=0, err_count=None,
                           stream=None) -> int:
    return _attn(_lib.dsa_sparse_attn_decode, q, q_dtype, q_scale, T, H, D,
                 rope_dim, pool, num_slots, layout, fp8_format, topk, K,
                 page_table, page_size, max_pages, num_seqs, token_seq,
                 seq_lens, softmax_scale, out, out_dtype, lse, workspace,
                 workspace_bytes, err_count, stream)


DSA_DECODE_SCRATCH_BYTES = 32 << 20


def dsa_sparse_attn_decode_noalloc(q, q_dtype, q_scale, T, H, D, rope_dim, pool,
                                   num_slots, layout, fp8_format, topk, K,
                                   page_table, page_size, max_pages, num_seqs,
                                   token_seq, seq_lens, softmax_scale, out,
                                   out_dtype, lse=None, err_count=None,
                                   stream=None) -> int:
    return _lib.dsa_sparse_attn_decode_noalloc(
        _p(q), q_dtype, _p(q_scale), T, H, D, rope_dim, _p(pool), num_slots,
        layout, fp8_format, _p(topk), K, _p(page_table), page_size, max_pages,
        num_seqs, _p(token_seq), _p(seq_lens), softmax_scale, _p(out), out_dtype,
        _p(lse), _p(err_count), _s(stream))


def dsa_sparse_attn_prefill(q, q_dtype, q_scale, T, H, D, rope_dim, pool,
                            num_slots, layout, fp8_format, topk, K, page_table,
                            page_size, max_pages, num_seqs, token_seq,
                            seq_lens, softmax_scale, out, out_dtype, lse=None,
                            workspace=None, workspace_bytes=0, err_count=None,
                            stream=None) -> int:
    return _attn(_lib.dsa_sparse_attn_prefill, q, q_dtype, q_scale, T, H, D,
                 rope_dim, pool, num_slots, layout, fp8_format, topk, K,
                 page_table, page_size, max_pages, num_seqs, token_seq,
                 seq_lens, softmax_scale, out, out_dtype, lse, workspace,
                 workspace_bytes, err_count, stream)


def dsa_topk_transform(topk, T, k_in, page_table, page_size, max_pages, num_seqs,
                       token_seq, seq_lens, num_slots, out_slots, k_out,
                       valid_count=None, err_count=None, stream=None) -> int:
    return _lib.dsa_topk_transform(_p(topk), T, k_in, _p(page_table), page_size,
                                   max_pages, num_seqs, _p(token_seq), _p(seq_lens),
                                   num_slots, _p(out_slots), k_out, _p(valid_count),
                                   _p(err_count), _s(stream))
