"""Full-size parity: the named workloads at their real sizes, through the same
entry points and launch configuration the benchmark times.  The device pool is
poisoned, every used page gets random finite codes, and the pages of the
compared tokens' sequences get oracle-written rows (also kept in a host pool
that is only materialised on those pages).  The writer step runs first; its
bytes are compared bit for bit.  The tiny decode and the decode batch (the
headline) are compared with the oracle token by token in full; the larger
configurations on at least 32 tokens that cover every token residue mod 8
(the XCD a token's workgroups run on), every head block and every split of
the top-k list.  Every token is checked for finiteness, and all-masked
tokens for exact zeros."""
import numpy as np
import pytest
import torch

import gpu_harness as G
import sparse_mla_attention_gather_amd as dsa
import workloads as W

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _materialise(orc, wl, seqs):
    """Host pool (lazily zero, only `seqs`' pages written) and the device pool
    (poison, random codes on every used page, the same rows on `seqs`' pages)."""
    R = wl.row_bytes
    host = np.zeros((wl.num_slots, R), np.uint8)
    slots = wl.page_slots(wl.used_pages(seqs))
    lat, sc = W.pool_content(wl.seed, len(slots), wl.layout)
    if wl.layout == W.BF16:
        host[slots] = np.ascontiguousarray(lat).view(np.uint8)
    elif wl.layout == W.RAW:
        tmp = np.zeros((len(slots), 512), np.uint8)
        orc.kv_write(lat, np.arange(len(slots)), tmp, W.RAW)
        host[slots] = tmp
    else:
        tmp = np.zeros((len(slots), 512), np.uint8)
        orc.kv_write(lat[:, :512], np.arange(len(slots)), tmp, W.RAW)
        host[slots, :512] = tmp
        host[slots, 512:528] = sc.view(np.uint8).reshape(len(slots), 16)
        if wl.layout == W.ROPE:
            host[slots, 528:] = np.ascontiguousarray(lat[:, 512:]).view(np.uint8)
    pool = torch.full((wl.num_slots, R), W.POISON, dtype=torch.uint8, device=G.DEV)
    used = torch.from_numpy(wl.page_slots(wl.used_pages())).to(G.DEV)
    gen = torch.Generator(device=G.DEV)
    gen.manual_seed(wl.seed)
    chunk = 1 << 20
    for i in range(0, used.numel(), chunk):
        u = used[i:i + chunk]
        r = torch.randint(0, 254, (u.numel(), 512), generator=gen, device=G.DEV,
                          dtype=torch.int32)
        rows = torch.empty((u.numel(), R), dtype=torch.uint8, device=G.DEV)
        rows[:, :512] = (r + (r >= 0x7F).int()).to(torch.uint8)
        if R == 1024:     # bf16 rows: N(0,1) values, not codes
            rows = torch.randn((u.numel(), 512), generator=gen, device=G.DEV).to(
                torch.bfloat16).contiguous().view(torch.uint8)
        if R in (528, 656):
            s = torch.exp2(torch.rand((u.numel(), 4), generator=gen, device=G.DEV) * 8 - 6)
            rows[:, 512:528] = s.contiguous().view(torch.uint8)
        if R == 656:
            rp = torch.randn((u.numel(), 64), generator=gen, device=G.DEV).to(torch.bfloat16)
            rows[:, 528:] = rp.contiguous().view(torch.uint8)
        pool[u] = rows
    pool[torch.from_numpy(slots).to(G.DEV)] = torch.from_numpy(host[slots]).to(G.DEV)
    return host, pool


def _writer_step(orc, wl, host, pool):
    ref_err = orc.kv_write(wl.kv_new, wl.slot_mapping, host, wl.layout)
    err = G.run_kv_write(wl.kv_new, wl.slot_mapping, pool, wl.layout)
    assert err == ref_err == 0
    sm = torch.from_numpy(wl.slot_mapping).to(G.DEV)
    got = G.host(pool[sm])
    assert np.array_equal(got, host[wl.slot_mapping]), "writer bytes differ"


def _sub(wl, idx):
    idx = np.asarray(idx)
    ts = np.asarray(idx, np.int32) if wl.token_seq is None else wl.token_seq[idx]
    return W.Workload(**{**wl.__dict__, "T": len(idx), "topk": wl.topk[idx],
                         "q": wl.q[idx], "token_seq": ts})


def _check(orc, wl, host, out, lse, sample, q8=None, scale=None, od=dsa.DSA_FP32):
    sub = _sub(wl, sample)
    qs = sub.q if q8 is None else q8[np.asarray(sample)]
    ref, ref_lse, err = orc.sparse_attn(qs, host, wl.layout, sub.topk,
                                        wl.softmax_scale, q_scale=scale,
                                        page_table=wl.page_table,
                                        page_size=wl.page_size,
                                        token_seq=sub.token_seq,
                                        seq_lens=wl.seq_lens)
    assert err == 0
    mx, mean = G.assert_attn_close(out[np.asarray(sample)], ref, od, where=wl.name)
    if lse is not None:
        G.assert_lse_close(lse[np.asarray(sample)], ref_lse, where=wl.name)
    print(f"{wl.name}: sampled tokens {list(sample)} max abs {mx:.2e} mean {mean:.2e}",
          flush=True)


def _decode_case(orc, wl, sample):
    print(f"full-size case {wl.name}: T={wl.T} H={wl.H} K={wl.K} sample={sample}",
          flush=True)
    seqs = sorted({int(t) if wl.token_seq is None else int(wl.token_seq[t]) for t in sample})
    host, pool = _materialise(orc, wl, seqs)
    _writer_step(orc, wl, host, pool)
    di = G.DevInputs(wl)
    for od in (dsa.DSA_FP32, dsa.DSA_BF16):
        out, lse, err = G.run_attn(di, pool, phase=0, out_dtype=od)
        assert err == 0
        assert np.all(np.isfinite(out)), "non-finite output"
        masked = np.all(wl.topk < 0, axis=1)
        assert np.all(out[masked] == 0) and np.all(lse[masked] == -np.inf)
        assert np.all(np.isfinite(lse[~masked]))
        _check(orc, wl, host, out, lse, sample, od=od)


def _spread_sample(T, n=32, extra=()):
    """n tokens of [0, T) spread over the batch, n / 8 of each residue mod 8
    (the XCD all of a token's workgroups run on), plus `extra`."""
    per = n // 8
    picks = set(extra)
    for r in range(8):
        cand = np.arange(r, T, 8)
        picks.update(int(x) for x in cand[np.linspace(0, len(cand) - 1, per).round().astype(int)])
    return sorted(picks)


def test_tiny_decode_full(orc):
    """The tiny decode configuration end to end: the writer fills the
    sequence's four pages of a poisoned 8-page pool, then every token and
    head is compared with the oracle (fp32 and bf16 output)."""
    wl = W.tiny_decode()
    print(f"full-size case {wl.name}: T={wl.T} H={wl.H} K={wl.K}", flush=True)
    slots = wl.page_slots(wl.used_pages())
    lat, _ = W.pool_content(wl.seed, len(slots), W.RAW)
    host = np.full((wl.num_slots, 512), W.POISON, np.uint8)
    assert orc.kv_write(lat, slots, host, W.RAW) == 0
    pool = torch.full((wl.num_slots, 512), W.POISON, dtype=torch.uint8, device=G.DEV)
    assert G.run_kv_write(lat, slots, pool, W.RAW) == 0
    assert np.array_equal(G.host(pool), host), "writer bytes differ"
    di = G.DevInputs(wl)
    for od in (dsa.DSA_FP32, dsa.DSA_BF16):
        out, lse, err = G.run_attn(di, pool, phase=0, out_dtype=od)
        assert err == 0
        _check(orc, wl, host, out, lse, list(range(wl.T)), od=od)


def test_decode_batch_full(orc):
    """The headline configuration, every one of its 64 tokens (all 16 heads,
    all four splits of each top-k list) against the oracle."""
    wl = W.decode_batch()
    _decode_case(orc, wl, list(range(wl.T)))


def test_bf16_decode_full(orc):
    """The decode batch's shape over 1024-byte bf16 rows."""
    wl = W.bf16_decode()
    _decode_case(orc, wl, [0, 21, 50, 63])


def test_rope_decode_full(orc):
    """The decode batch's shape over 656-byte RoPE rows."""
    wl = W.rope_decode()
    _decode_case(orc, wl, [0, 13, 32, 63])


def test_scaled_decode_full(orc):
    wl = W.scaled_decode()
    empty = int(np.nonzero(np.all(wl.topk < 0, axis=1))[0][0])
    _decode_case(orc, wl, _spread_sample(wl.T, 32, extra=(empty,)))


def test_mixed_decode_full(orc):
    """Both 32-head blocks of every compared token, over all three top-k
    widths."""
    wl = W.mixed_decode()
    # the longest sequences put byte offsets of their pages beyond 4 GiB
    far = int(np.argmax(wl.page_table.max(axis=1)))
    sample = _spread_sample(wl.T, 32, extra=(far,))
    widths = {int(np.sum(wl.topk[t] >= 0)) for t in sample}
    assert widths == {1024, 1536, 2048}
    _decode_case(orc, wl, sample)


def test_q8_prefill_full(orc):
    """Writer -> query cast -> prefill over the 16384-token prefix plus the
    4096 freshly written rows, the configuration the prefill bench runs."""
    wl = W.q8_prefill()
    print(f"full-size case {wl.name}: T={wl.T} H={wl.H} K={wl.K}", flush=True)
    host = np.zeros((wl.num_slots, 512), np.uint8)
    prefix = 16384
    pos = np.arange(prefix, dtype=np.int64)
    pre_slots = wl.page_table[0][pos // 64].astype(np.int64) * 64 + pos % 64
    lat, _ = W.pool_content(wl.seed, prefix, W.RAW)
    orc.kv_write(lat, pre_slots, host, W.RAW)
    pool = torch.full((wl.num_slots, 512), W.POISON, dtype=torch.uint8, device=G.DEV)
    pool[torch.from_numpy(pre_slots).to(G.DEV)] = torch.from_numpy(host[pre_slots]).to(G.DEV)
    _writer_step(orc, wl, host, pool)
    di = G.DevInputs(wl)
    q8_d, sc_d = G.run_quantize(di.q)
    s_ref = orc.q_scale(wl.q)
    q8_ref = orc.q_quantize(wl.q, s_ref)
    assert G.host(sc_d)[0].view(np.uint32) == np.float32(s_ref).view(np.uint32)
    assert np.array_equal(G.host(q8_d), q8_ref)
    out, lse, err = G.run_attn(di, pool, phase=1, q=q8_d, q_scale=sc_d)
    assert err == 0
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    _check(orc, wl, host, out, lse,
           sorted(set(_spread_sample(wl.T, 32)) | {0, 1, 126, 127, 128, 2047, 4095}),
           q8=q8_ref, scale=s_ref)
