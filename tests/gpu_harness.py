"""Device-side plumbing for the GPU parity tests: upload a workload, call the
C ABI through the Python binding, bring results back.  Parity tolerances live
here too.  Inputs come from ``workloads`` (and, for pool bytes, from the
oracle's writer); nothing here computes any part of the method."""
from __future__ import annotations

import numpy as np
import torch

import sparse_mla_attention_gather_amd as dsa
import workloads as W

DEV = torch.device("cuda:0")

# Attention parity bar (fp32 output, against FP64 on identical dequantised
# inputs): max abs 2e-2, mean abs 2e-3.
MAX_ABS = 2e-2
MEAN_ABS = 2e-3
LSE_ABS = 1e-3


def dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(DEV)
    return torch.from_numpy(a).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def bf16_bits_host(t: torch.Tensor) -> np.ndarray:
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def check(st: int):
    assert st == 0, dsa.dsa_status_string(st)


class DevInputs:
    """The index-side tensors of a workload on the device."""

    def __init__(self, wl: W.Workload):
        self.wl = wl
        self.topk = dev(wl.topk.astype(np.int32))
        self.page_table = None if wl.page_table is None else dev(wl.page_table)
        self.seq_lens = None if wl.seq_lens is None else dev(wl.seq_lens)
        self.token_seq = None if wl.token_seq is None else dev(wl.token_seq)
        self.q = dev(wl.q)
        self.num_seqs = 0 if wl.page_table is None and wl.seq_lens is None else (
            wl.page_table.shape[0] if wl.page_table is not None else len(wl.seq_lens))
        self.max_pages = 0 if wl.page_table is None else wl.page_table.shape[1]


def run_attn(di: DevInputs, pool_dev: torch.Tensor, *, phase: int = 0,
             out_dtype: int = dsa.DSA_FP32, q=None, q_scale=None,
             lse: bool = True, topk=None, stream=None):
    """Returns (out float32 [T,H,512], lse float32 [T,H] or None, err_count)."""
    wl = di.wl
    T, H, K = wl.T, wl.H, (wl.K if topk is None else topk.shape[1])
    out = torch.empty((T, H, 512), dtype=torch.float32 if out_dtype == dsa.DSA_FP32
                      else torch.bfloat16, device=DEV)
    lse_t = torch.empty((T, H), dtype=torch.float32, device=DEV) if lse else None
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    wsb = dsa.dsa_attn_workspace_bytes(T, H, K, phase)
    ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=DEV)
    fn = dsa.dsa_sparse_attn_decode if phase == 0 else dsa.dsa_sparse_attn_prefill
    fp8q = q_scale is not None
    check(fn(di.q if q is None else q, dsa.DSA_FP8_E4M3FN if fp8q else dsa.DSA_BF16,
             q_scale, T, H, 512, wl.rope_dim, pool_dev, pool_dev.shape[0], wl.layout,
             dsa.DSA_FP8_E4M3FN, di.topk if topk is None else topk, K,
             di.page_table, wl.page_size, di.max_pages, di.num_seqs,
             di.token_seq, di.seq_lens, wl.softmax_scale, out, out_dtype,
             lse_t, ws, wsb, err, stream))
    torch.cuda.synchronize()
    o = out.float().cpu().numpy()
    return o, (None if lse_t is None else host(lse_t)), int(err.item())


def run_kv_write(kv: np.ndarray, slot_mapping: np.ndarray, pool_dev: torch.Tensor,
                 layout: int) -> int:
    kv_d = dev(kv)
    sm = dev(slot_mapping.astype(np.int64))
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    check(dsa.dsa_kv_write(kv_d, kv.shape[0], kv.shape[1], dsa.DSA_BF16, 512,
                           64 if layout == W.ROPE else 0,
                           sm, pool_dev, pool_dev.shape[0], layout,
                           dsa.DSA_FP8_E4M3FN, err))
    torch.cuda.synchronize()
    return int(err.item())


def run_quantize(q_dev: torch.Tensor, scale_given=None):
    n = q_dev.numel()
    q8 = torch.empty(q_dev.shape, dtype=torch.uint8, device=DEV)
    sc = torch.empty(1, dtype=torch.float32, device=DEV)
    if scale_given is not None:
        sc.fill_(float(scale_given))
    wsb = dsa.dsa_quantize_q_workspace_bytes(n)
    ws = torch.empty(max(wsb, 4), dtype=torch.uint8, device=DEV)
    check(dsa.dsa_quantize_q_fp8(q_dev, n, dsa.DSA_BF16, q8, sc,
                                 int(scale_given is not None), dsa.DSA_FP8_E4M3FN,
                                 ws, wsb))
    torch.cuda.synchronize()
    return q8, sc


def assert_attn_close(got, ref, out_dtype=dsa.DSA_FP32, where=""):
    assert got.shape == ref.shape
    assert np.all(np.isfinite(got)), f"{where}: non-finite output"
    err = np.abs(got.astype(np.float64) - ref)
    if out_dtype == dsa.DSA_FP32:
        tol = np.full_like(ref, MAX_ABS)
        mean_tol = MEAN_ABS
    else:
        # bf16 output: the fp32 bar plus the output's own rounding (half an
        # ulp of bf16's 8-bit significand at the reference's magnitude)
        half_ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 8)
        tol = MAX_ABS + half_ulp
        mean_tol = MEAN_ABS + float(np.mean(half_ulp))
    bad = err > tol
    assert not bad.any(), (f"{where}: {bad.sum()} outputs beyond tolerance, "
                           f"max err {err.max():.3e}")
    assert err.mean() <= mean_tol, f"{where}: mean abs err {err.mean():.3e}"
    return float(err.max()), float(err.mean())


def assert_lse_close(got, ref, where=""):
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), fin), f"{where}: lse finiteness"
    assert np.all(got[~fin] == ref[~fin]), f"{where}: lse -inf"
    if fin.any():
        e = np.max(np.abs(got[fin] - ref[fin]))
        assert e <= LSE_ABS, f"{where}: lse err {e:.3e}"
