"""Throughput of the DSA sparse-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = one pass of the hot path over one batch: the fused writer appends
each sequence's newest latent to the paged FP8 pool, then sparse attention
runs over every token's top-k rows (decode: split top-k + merge kernel;
the Q8 prefill workload also casts the query to FP8 first).  Inputs are
resident in HBM before the timed region.  Consecutive steps rotate over
several independent layer pools (as consecutive layers of a model do) so
that at least 1 GiB of rows is gathered per rotation and the 256 MB
Infinity Cache cannot serve the step from the previous visit.

Prints ONE JSON line.  `value` is query tokens per second of the whole step
loop (W warm-up steps, then one untimed step per layer pool the warm-up did
not reach, then K timed steps with nothing else on the stream).  After the
timed loop, a timing pass runs --timing-calls more steps (at least 20) in
which the writer, the query cast and the attention call are each bracketed
by HIP events on the launch stream; `roofline` relates the attention call's
algorithmic bytes (decode: gathered row bytes) or FLOPs (prefill) to its mean
duration there, and the median, p10 and p90 are reported beside it.
`cpu_baseline` times the CPU oracle on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_TFLOPS = 2500.0       # dense bf16/f16 matrix peak, published
MFMA_FP8_TFLOPS = 5000.0        # dense fp8 matrix peak, published
METRIC = "query tok/s + gathered-KV GB/s (% HBM peak), decode H=16 top-k=2048"
MIN_TIMING_CALLS = 20           # event-timed attention calls, at least
# clock cycles of stream spin per bracketed step (about 250 us at 2 GHz, well
# above the host's cost of enqueueing one step)
SPIN_CYCLES_PER_STEP = 500_000


def spin(cycles: int) -> None:
    """A kernel that keeps the current stream busy for about `cycles` clock
    cycles (PyTorch's own spin kernel; skipped where this build lacks it)."""
    import torch
    fn = getattr(torch.cuda, "_sleep", None)
    if fn is not None:
        fn(int(cycles))


class TimingEvent:
    """A HIP event used only to measure time, recorded on torch's current
    stream (the stream the library launches on).  It is created with
    hipEventDisableSystemFence through the HIP runtime torch has loaded: the
    runtime documents that flag for timing-only events, whose recording then
    does not write back and invalidate the caches around the timed work (a
    default event's system-scope fence does, and its cost lands partly inside
    the bracket).  Same interface as torch.cuda.Event: record(),
    elapsed_time(end) in ms."""
    DISABLE_SYSTEM_FENCE = 0x20000000
    _lib = None

    @classmethod
    def lib(cls):
        if cls._lib is None:
            import ctypes
            import torch
            lib = ctypes.CDLL(os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so"))
            P = ctypes.c_void_p
            lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(P), ctypes.c_uint]
            lib.hipEventRecord.argtypes = [P, P]
            lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), P, P]
            lib.hipEventDestroy.argtypes = [P]
            for f in (lib.hipEventCreateWithFlags, lib.hipEventRecord,
                      lib.hipEventElapsedTime, lib.hipEventDestroy):
                f.restype = ctypes.c_int
            cls._lib = lib
        return cls._lib

    def __init__(self):
        import ctypes
        self._h = ctypes.c_void_p()
        rc = self.lib().hipEventCreateWithFlags(ctypes.byref(self._h), self.DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")

    def record(self):
        import ctypes
        import torch
        rc = self.lib().hipEventRecord(self._h, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_time(self, end) -> float:
        import ctypes
        ms = ctypes.c_float()
        rc = self.lib().hipEventElapsedTime(ctypes.byref(ms), self._h, end._h)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def __del__(self):
        if self._lib is not None and self._h:
            self._lib.hipEventDestroy(self._h)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode_batch",
                    choices=["decode_batch", "scaled_decode", "mixed_decode",
                             "q8_prefill", "tiny_decode", "rope_decode", "bf16_decode"])
    ap.add_argument("--layers", type=int, default=0,
                    help="layer pools to rotate over (0 = enough for 1 GiB)")
    ap.add_argument("--out-dtype", default="bf16", choices=["bf16", "fp32"])
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU baseline")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 1 GiB device copy (counter scaling)")
    ap.add_argument("--timing-calls", type=int, default=200,
                    help="event-timed steps after the timed loop (at least 20)")
    ap.add_argument("--op", default="attention", choices=["attention", "transform"],
                    help="transform: time the index transform alone on the "
                         "workload's top-k rows (page table -> compacted slots)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this library runs on exactly one GPU; --gpus N with N > 1 "
              "is not supported (no sharding or collectives on this path)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import sparse_mla_attention_gather_amd as dsa
    import workloads as W

    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    wl = W.NAMED[args.workload]()
    if args.op == "transform":
        return bench_transform(args, wl, dev)
    T, H, K, R = wl.T, wl.H, wl.K, wl.row_bytes
    rope = wl.rope_dim                                 # RoPE values per row (656-byte rows)
    prefill = wl.q_fp8
    phase = 1 if prefill else 0
    out_dtype = dsa.DSA_BF16 if args.out_dtype == "bf16" else dsa.DSA_FP32

    valid_entries = int(np.sum(wl.topk >= 0))
    gathered = valid_entries * R                       # algorithmic bytes / call
    # the same with each token's repeated entries counted once
    unique_entries = int(sum(np.unique(r[r >= 0]).size for r in wl.topk))
    unique_gathered = unique_entries * R
    flops = 4.0 * H * 512 * valid_entries              # QK + PV per call
    if args.layers > 0:
        layers = args.layers
    else:
        layers = max(2, min(16, math.ceil((1 << 30) / max(gathered, 1))))
        if prefill:
            layers = 2
    print(f"bench: {wl.name} T={T} H={H} K={K} rows={R}B valid={valid_entries} "
          f"layers={layers}", file=sys.stderr, flush=True)

    # ---- device inputs (shared index tensors, per-layer pools and queries)
    topk = torch.from_numpy(wl.topk).to(dev)
    pt = torch.from_numpy(wl.page_table).to(dev)
    sl = torch.from_numpy(wl.seq_lens).to(dev)
    ts = None if wl.token_seq is None else torch.from_numpy(wl.token_seq).to(dev)
    num_seqs, max_pages = wl.page_table.shape
    # the step's writer call: the workload's new latent rows (none for the
    # tiny parity case, whose step is the attention alone)
    n_new = 0 if wl.kv_new is None else wl.kv_new.shape[0]
    if n_new:
        kv_new = torch.from_numpy(wl.kv_new.view(np.int16)).to(dev)
        slot_map = torch.from_numpy(wl.slot_mapping).to(dev)
    used = torch.from_numpy(wl.page_slots(wl.used_pages())).to(dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(wl.seed)
    pools, qs = [], []
    for layer in range(layers):
        pool = torch.full((wl.num_slots, R), 0xFF, dtype=torch.uint8, device=dev)
        # fill every used page through the writer from N(0,1) latents
        chunk = 1 << 18
        for i in range(0, used.numel(), chunk):
            sl_i = used[i:i + chunk]
            lat = torch.randn((sl_i.numel(), 512 + rope), generator=gen, device=dev,
                              dtype=torch.float32).to(torch.bfloat16)
            dsa.check(dsa.dsa_kv_write(lat, sl_i.numel(), 512 + rope, dsa.DSA_BF16, 512, rope,
                                       sl_i, pool, wl.num_slots, wl.layout,
                                       dsa.DSA_FP8_E4M3FN))
        pools.append(pool)
        qs.append(torch.randn((T, H, 512 + rope), generator=gen, device=dev,
                              dtype=torch.float32).to(torch.bfloat16))
    torch.cuda.synchronize()

    out = torch.empty((T, H, 512), device=dev,
                      dtype=torch.bfloat16 if out_dtype == dsa.DSA_BF16 else torch.float32)
    lse = torch.empty((T, H), device=dev, dtype=torch.float32)
    wsb = dsa.dsa_attn_workspace_bytes(T, H, K, phase)
    ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=dev)
    q8 = torch.empty((T, H, 512), dtype=torch.uint8, device=dev)
    q_scale = torch.empty(1, dtype=torch.float32, device=dev)
    qwsb = dsa.dsa_quantize_q_workspace_bytes(T * H * 512)
    qws = torch.empty(max(qwsb, 4), dtype=torch.uint8, device=dev)
    attn = dsa.dsa_sparse_attn_prefill if prefill else dsa.dsa_sparse_attn_decode

    def step(i, ev=None):
        """One pass of the hot path on layer pool i % layers; `ev` (four
        timing events) brackets the writer, the query cast and the attention
        call."""
        layer = i % layers
        pool = pools[layer]
        if ev is not None:
            ev[0].record()
        if n_new:
            dsa.check(dsa.dsa_kv_write(kv_new, n_new, 512 + rope, dsa.DSA_BF16, 512, rope,
                                       slot_map, pool, wl.num_slots, wl.layout,
                                       dsa.DSA_FP8_E4M3FN))
        if ev is not None:
            ev[1].record()
        if prefill:
            dsa.check(dsa.dsa_quantize_q_fp8(qs[layer], T * H * 512, dsa.DSA_BF16,
                                             q8, q_scale, 0, dsa.DSA_FP8_E4M3FN,
                                             qws, qwsb))
            q, qd, qsc = q8, dsa.DSA_FP8_E4M3FN, q_scale
        else:
            q, qd, qsc = qs[layer], dsa.DSA_BF16, None
        if ev is not None:
            ev[2].record()
        dsa.check(attn(q, qd, qsc, T, H, 512, rope, pool, wl.num_slots, wl.layout,
                       dsa.DSA_FP8_E4M3FN, topk, K, pt, wl.page_size, max_pages,
                       num_seqs, ts, sl, wl.softmax_scale, out, out_dtype, lse,
                       ws, wsb, None))
        if ev is not None:
            ev[3].record()

    for i in range(args.warmup):
        step(i)
    # every layer pool meets the kernels once before the timed loop, whatever
    # the warm-up count (first touches of a pool cost page-table walks)
    pool_warm = list(range(args.warmup, layers))
    for i in pool_warm:
        step(i)
    first = max(args.warmup, layers)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(first + i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    elapsed = t1 - t0
    ms_per_step = elapsed * 1e3 / args.steps
    tok_s = T * args.steps / elapsed

    # timing pass: the same steps, continuing the pool rotation, with the
    # writer, the query cast and the attention call each bracketed by events
    # (a pair of events costs the stream time of its own, so the throughput
    # loop above carries none)
    n_ev = max(MIN_TIMING_CALLS, args.timing_calls)
    events = [tuple(TimingEvent() for _ in range(4)) for _ in range(n_ev)]
    torch.cuda.synchronize()
    # a spin kernel ahead of the bracketed steps keeps the stream busy while
    # the host enqueues them, so that every bracket holds GPU time alone
    # (on an idle stream a start event passes before the host has launched
    # the kernels it brackets, and the launch cost lands inside)
    spin(n_ev * SPIN_CYCLES_PER_STEP)
    for j in range(n_ev):
        step(first + args.steps + j, events[j])
    torch.cuda.synchronize()
    writer_ms = np.array([e[0].elapsed_time(e[1]) for e in events])
    qcast_ms = np.array([e[1].elapsed_time(e[2]) for e in events])
    attn_ms = np.array([e[2].elapsed_time(e[3]) for e in events])
    attn_avg_s = float(np.mean(attn_ms)) * 1e-3

    traffic = committed_traffic(wl.name)
    if prefill:
        # QK^T runs on the FP8 matrix cores, PV on the f16 ones (half of the
        # FLOPs each): the peak is the rate at which both halves would finish
        # together at their own dtype's peak
        peak = flops / (0.5 * flops / MFMA_FP8_TFLOPS + 0.5 * flops / MFMA_BF16_TFLOPS)
        achieved = flops / attn_avg_s / 1e12
        roofline = {"bound": "mfma", "achieved": achieved, "peak": peak,
                    "unit": "TFLOP/s", "frac": achieved / peak,
                    "traffic": traffic}
    else:
        achieved = gathered / attn_avg_s / 1e9
        roofline = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS,
                    "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic}

    if args.copy_calibration:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(wl, args.cpu_seconds)

    rec = {
        "metric": METRIC,
        "value": tok_s,
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8" if prefill else "bf16",
        "data": "synthetic",
        "config": {
            "workload": wl.name, "T": T, "H": H, "top_k": K,
            "valid_entries": valid_entries, "kv_row_bytes": R,
            "pool_slots": wl.num_slots, "page_size": wl.page_size,
            "q": "fp8_e4m3fn per-tensor scale" if prefill else "bf16",
            "out": args.out_dtype, "layer_pools": layers,
        },
        "attn_us": attn_avg_s * 1e6,
        "attn_us_median": float(np.median(attn_ms)) * 1e3,
        "attn_us_p10_p90": [float(np.percentile(attn_ms, 10)) * 1e3,
                            float(np.percentile(attn_ms, 90)) * 1e3],
        "attn_timed_calls": int(len(attn_ms)),
        "attn_tok_s": T / attn_avg_s,
        "writer_us": float(np.mean(writer_ms)) * 1e3 if n_new else None,
        "writer_rows": n_new,
        "q_cast_us": float(np.mean(qcast_ms)) * 1e3 if prefill else None,
        "pool_warm_calls": len(pool_warm),
        "gathered_GBps": gathered / attn_avg_s / 1e9,
        "gathered_bytes_per_call": gathered,
        "unique_gathered_bytes_per_call": unique_gathered,
        "unique_gathered_GBps": unique_gathered / attn_avg_s / 1e9,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


def bench_transform(args, wl, dev):
    """The index transform alone: each step resolves and compacts every
    top-k row of the workload (same rows each step).  Algorithmic bytes per
    call: the int32 top-k read, the int32 slots and counts written; the
    page-table words are read once per entry but come from cache."""
    import torch

    import sparse_mla_attention_gather_amd as dsa

    T, K = wl.topk.shape
    d = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(dev)
    topk, pt, ts, sl = d(wl.topk), d(wl.page_table), d(wl.token_seq), d(wl.seq_lens)
    num_seqs, max_pages = (0, 0) if wl.page_table is None else wl.page_table.shape
    out = torch.empty((T, K), dtype=torch.int32, device=dev)
    counts = torch.empty(T, dtype=torch.int32, device=dev)

    def call():
        dsa.check(dsa.dsa_topk_transform(topk, T, K, pt, wl.page_size, max_pages, num_seqs,
                                         ts, sl, wl.num_slots, out, K, counts, None))

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        call()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    n_ev = max(MIN_TIMING_CALLS, args.timing_calls)
    events = [(TimingEvent(), TimingEvent()) for _ in range(n_ev)]
    spin(n_ev * SPIN_CYCLES_PER_STEP)   # as in the attention timing pass
    for ev in events:
        ev[0].record()
        call()
        ev[1].record()
    torch.cuda.synchronize()
    call_ms = np.array([a.elapsed_time(b) for a, b in events])
    call_s = float(np.mean(call_ms)) * 1e-3
    nbytes = 4 * T * K + 4 * T * K + 4 * T
    achieved = nbytes / call_s / 1e9
    rec = {
        "metric": "top-k entries/s, index transform (page table -> compacted slots)",
        "value": T * K * args.steps / elapsed,
        "unit": "entries/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": elapsed * 1e3 / args.steps,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "int32", "data": "synthetic",
        "config": {"workload": f"topk_transform/{wl.name}", "T": T, "k_in": K, "k_out": K,
                   "page_size": wl.page_size},
        "transform_us": call_s * 1e6,
        "transform_us_median": float(np.median(call_ms)) * 1e3,
        "transform_timed_calls": int(len(call_ms)),
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": committed_traffic(wl.name, "topk_transform",
                                                  "topk_transform.hip")},
        "cpu_baseline": None,
    }
    if not args.no_cpu:
        import oracle
        orc = oracle.get()
        n, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < min(args.cpu_seconds, 5.0):
            orc.topk_transform(wl.topk, wl.num_slots, K, page_table=wl.page_table,
                               page_size=wl.page_size, token_seq=wl.token_seq,
                               seq_lens=wl.seq_lens)
            n += 1
        rec["cpu_baseline"] = {"value": T * K * n / (time.perf_counter() - t0),
                               "unit": "entries/s", "cores": 1, "kind": "oracle",
                               "sample": f"{n} whole transform(s) of the {wl.name} rows",
                               **host_description()}
    print(json.dumps(rec), flush=True)


def committed_traffic(workload, op="attn", source="attn.hip"):
    """HBM bytes of one call as measured by the rocprofv3 counter runs
    summarised in profiles/<op>_<workload>_traffic.txt (FETCH_SIZE and
    WRITE_SIZE per dispatch, scaled by what the same counters read for a 1 GiB
    device copy), or None when there is no such summary or the kernel source
    has changed since it was taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{op}_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if line.startswith("#") or not line.strip():
            continue
        k, v = line.split()[:2]
        fields[k] = v
    h = hashlib.sha256()
    for f in (f"sparse_mla_attention_gather_amd/csrc/{source}",
              "sparse_mla_attention_gather_amd/csrc/common.h"):
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    if fields.get("kernel_source_sha256") != h.hexdigest():
        return None
    return float(fields["traffic_bytes_per_call"])


def host_description():
    """The host the oracle runs on: logical CPUs of the machine and of this
    process, and the CPU model."""
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    avail = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return {"nproc": avail, "machine_cpus": os.cpu_count(), "cpu_model": model}


def cpu_baseline(wl, budget_s):
    """The oracle (as it stands) on a bounded sample of the same workload:
    whole steps (writer on the new rows + attention for every token of the
    batch) over a host pool whose used pages hold random finite FP8 codes,
    repeated until about `budget_s` seconds have passed."""
    import oracle
    import workloads as W

    orc = oracle.get()
    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    cores = max(1, min(cores, 16))      # the host-core share of one GPU
    R = wl.row_bytes
    rng = np.random.default_rng(wl.seed + 1000)
    T_s = wl.T
    if wl.q_fp8:
        T_s = min(wl.T, 64)     # prefill: a token slice of the batch
    pool = np.zeros((wl.num_slots, R), np.uint8)
    slots = wl.page_slots(wl.used_pages())
    pool[slots, :512] = W.random_fp8_codes(rng, (len(slots), 512))
    if R in (528, 656):
        pool[slots, 512:528] = W.log_uniform_scales(rng, len(slots)).view(np.uint8)
    if R == 656:
        pool[slots, 528:] = W.normal_bf16(rng, (len(slots), 64)).view(np.uint8)
    if R == 1024:
        pool[slots] = W.normal_bf16(rng, (len(slots), 512)).view(np.uint8)
    sel = slice(0, T_s)
    q = wl.q[sel]
    q8 = scale = None
    steps, tokens, t_total = 0, 0, 0.0
    while True:
        t0 = time.perf_counter()
        if wl.kv_new is not None:
            orc.kv_write(wl.kv_new, wl.slot_mapping, pool, wl.layout)
        if wl.q_fp8:
            scale = orc.q_scale(q)
            q8 = orc.q_quantize(q, scale)
        orc.sparse_attn(q if q8 is None else q8, pool, wl.layout, wl.topk[sel],
                        wl.softmax_scale, q_scale=scale, page_table=wl.page_table,
                        page_size=wl.page_size,
                        token_seq=None if wl.token_seq is None else wl.token_seq[sel],
                        seq_lens=wl.seq_lens, nthreads=cores)
        t_total += time.perf_counter() - t0
        steps += 1
        tokens += T_s
        if t_total >= budget_s or steps >= 500:
            break
    return {"value": tokens / t_total, "unit": "tok/s", "cores": cores,
            "kind": "oracle", **host_description(),
            "sample": f"{steps} step(s) of {wl.name}: writer on the "
                      f"{0 if wl.kv_new is None else wl.kv_new.shape[0]} "
                      f"new rows + FP64 attention for {T_s} tokens x {wl.H} heads x "
                      f"top-k {wl.K}; {t_total:.1f} s on {cores} threads"}


if __name__ == "__main__":
    main()
