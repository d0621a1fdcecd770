"""The hot path as a pipeline, on the GPU.

* Graph replay of the prefill pipeline: the fused writer, the FP8 query cast
  and the prefill attention are captured once in one HIP graph and replayed
  after the new latent rows, the query, the supplied query scale and the
  top-k indices have been changed in place; every replay is compared with the
  oracle ("[DSA] Support group-scaled FP8 NoPE KV reads for CUDA TileLang",
  Accuracy Tests: graph replay with changing indices, queries and scale
  data).  Eager work and synchronisations run between the replays.  16 and
  32 heads (the 16- and 32-head block forms of the attention).
* Context-parallel merge on one GPU: the pages name an attention
  context-parallel split whose partial results are merged by their
  log-sum-exp ("extend CUDA TileLang raw FP8 KV path", Modifications, where
  attn_cp_size is validated).  One decode call is split into n calls, each
  seeing only the entries whose pages fall in its own page range (the others
  set to -1); their (out, lse) are merged with o = sum_r e^(lse_r - lse) o_r,
  lse = log sum_r e^(lse_r), and compared with the single call and with the
  oracle.  This checks the lse output as the input of a later merge, which is
  what a rank's partial result is under that split."""
import numpy as np
import pytest
import torch

import gpu_harness as G
import oracle_pins as P
import sparse_mla_attention_gather_amd as dsa
import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("given_scale", [False, True], ids=["amax_scale", "given_scale"])
@pytest.mark.parametrize("H", [16, 32], ids=["h16", "h32"])
def test_graph_replay_prefill_pipeline(orc, given_scale, H):
    # (32 heads: the 32-head block form of the attention)
    prefix, T, K = 200, 300, 256
    wl = W.q8_prefill(seed=45, prefix=prefix, T=T, H=H, K=K, num_slots=1 << 14)
    print(f"graph replay prefill pipeline: T={T} H={H} K={K} given_scale={given_scale}",
          flush=True)
    # the prefix rows, written once by the oracle's writer; the graph's
    # writer appends the T new rows on every replay
    base_pool = np.full((wl.num_slots, 512), W.POISON, np.uint8)
    lat, _ = W.pool_content(wl.seed, prefix, W.RAW)
    pos = np.arange(prefix, dtype=np.int64)
    pre_slots = wl.page_table[0][pos // 64].astype(np.int64) * 64 + pos % 64
    orc.kv_write(lat, pre_slots, base_pool, W.RAW)

    pool = G.dev(base_pool)
    kv_new = G.dev(wl.kv_new)
    slot_map = G.dev(wl.slot_mapping)
    di = G.DevInputs(wl)
    q8 = torch.empty((T, H, 512), dtype=torch.uint8, device=G.DEV)
    q_scale = torch.ones(1, dtype=torch.float32, device=G.DEV)
    qwsb = dsa.dsa_quantize_q_workspace_bytes(T * H * 512)
    qws = torch.empty(max(qwsb, 4), dtype=torch.uint8, device=G.DEV)
    out = torch.empty((T, H, 512), dtype=torch.float32, device=G.DEV)
    lse = torch.empty((T, H), dtype=torch.float32, device=G.DEV)
    wsb = dsa.dsa_attn_workspace_bytes(T, H, K, 1)
    ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=G.DEV)
    err = torch.zeros(1, dtype=torch.int32, device=G.DEV)

    def pipeline():
        G.check(dsa.dsa_kv_write(kv_new, T, 512, dsa.DSA_BF16, 512, 0, slot_map, pool,
                                 wl.num_slots, dsa.DSA_KV_RAW_FP8_512, dsa.DSA_FP8_E4M3FN, err))
        G.check(dsa.dsa_quantize_q_fp8(di.q, T * H * 512, dsa.DSA_BF16, q8, q_scale,
                                       int(given_scale), dsa.DSA_FP8_E4M3FN, qws, qwsb))
        G.check(dsa.dsa_sparse_attn_prefill(
            q8, dsa.DSA_FP8_E4M3FN, q_scale, T, H, 512, 0, pool, wl.num_slots,
            dsa.DSA_KV_RAW_FP8_512, dsa.DSA_FP8_E4M3FN, di.topk, K, di.page_table,
            wl.page_size, di.max_pages, di.num_seqs, di.token_seq, di.seq_lens,
            wl.softmax_scale, out, dsa.DSA_FP32, lse, ws, wsb, err))

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        pipeline()                                # warm-up outside capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pipeline()

    for it in range(3):
        # new rows, queries, indices (and supplied scale), same geometry
        w2 = W.q8_prefill(seed=46 + it, prefix=prefix, T=T, H=H, K=K, num_slots=1 << 14)
        scale = None
        if given_scale:
            scale = np.float32(orc.q_scale(w2.q) * np.float32([0.8, 1.3, 2.0][it]))
            q_scale.fill_(float(scale))
        kv_new.copy_(torch.from_numpy(w2.kv_new.view(np.int16)))
        di.q.copy_(torch.from_numpy(w2.q.view(np.int16)))
        di.topk.copy_(torch.from_numpy(w2.topk))
        err.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()

        ref_pool = base_pool.copy()
        assert orc.kv_write(w2.kv_new, wl.slot_mapping, ref_pool, W.RAW) == 0
        assert np.array_equal(G.host(pool), ref_pool), f"replay {it}: writer bytes"
        s_ref = orc.q_scale(w2.q) if scale is None else scale
        assert G.host(q_scale)[0].view(np.uint32) == np.float32(s_ref).view(np.uint32)
        q8_ref = orc.q_quantize(w2.q, s_ref)
        assert np.array_equal(G.host(q8), q8_ref), f"replay {it}: query codes"
        ref, ref_lse, ref_err = orc.sparse_attn(q8_ref, ref_pool, W.RAW, w2.topk,
                                                wl.softmax_scale, q_scale=s_ref,
                                                page_table=wl.page_table,
                                                page_size=wl.page_size,
                                                token_seq=wl.token_seq, seq_lens=wl.seq_lens)
        assert int(err.item()) == ref_err == 0
        G.assert_attn_close(G.host(out), ref, where=f"replay {it}")
        G.assert_lse_close(G.host(lse), ref_lse, where=f"replay {it}")
        # eager work between replays
        _ = (out.sum() + 1).item()


def _lse_merge(outs, lses):
    """o = sum_r e^(lse_r - lse) o_r, lse = log sum_r e^(lse_r), in FP64; a
    part with lse_r = -inf carries no weight; all parts empty -> 0, -inf."""
    L = np.stack([l.astype(np.float64) for l in lses])          # [n, T, H]
    O = np.stack([o.astype(np.float64) for o in outs])          # [n, T, H, 512]
    m = np.max(L, axis=0)
    fin = np.isfinite(m)
    w = np.where(np.isfinite(L), np.exp(L - np.where(fin, m, 0.0)), 0.0)
    tot = w.sum(axis=0)
    lse = np.where(fin, m + np.log(np.where(fin, tot, 1.0)), -np.inf)
    o = np.where(fin[..., None], (w[..., None] * O).sum(axis=0)
                 / np.where(fin, tot, 1.0)[..., None], 0.0)
    return o, lse


@pytest.mark.parametrize("layout", [W.RAW, W.SCALED], ids=["raw", "scaled"])
@pytest.mark.parametrize("n", [2, 3])
@pytest.mark.parametrize("H", [16, 32], ids=["h16", "h32"])
def test_context_parallel_lse_merge(orc, layout, n, H):
    wl = W.small(601 + n, T=6, H=H, K=1024, layout=layout, seq_len=3000, page_size=64,
                 all_masked=(4,))
    pool = P.build_pool(orc, wl)
    pool_d = G.dev(pool)
    di = G.DevInputs(wl)
    ref, ref_lse, _ = orc.sparse_attn(wl.q, pool, wl.layout, wl.topk, wl.softmax_scale,
                                      page_table=wl.page_table, page_size=wl.page_size,
                                      token_seq=wl.token_seq, seq_lens=wl.seq_lens)
    full, full_lse, err = G.run_attn(di, pool_d, phase=0)
    assert err == 0
    # rank r owns the physical pages [r P / n, (r + 1) P / n)
    n_pages = wl.num_slots // wl.page_size
    valid = wl.topk >= 0
    page = np.where(valid, wl.page_table[wl.token_seq[:, None],
                                         np.where(valid, wl.topk, 0) // wl.page_size], -1)
    outs, lses = [], []
    for r in range(n):
        lo, hi = r * n_pages // n, (r + 1) * n_pages // n
        mine = valid & (page >= lo) & (page < hi)
        assert mine.any()
        topk_r = G.dev(np.where(mine, wl.topk, -1).astype(np.int32))
        o_r, l_r, err = G.run_attn(di, pool_d, phase=0, topk=topk_r)
        assert err == 0
        outs.append(o_r)
        lses.append(l_r)
    merged, merged_lse = _lse_merge(outs, lses)
    G.assert_attn_close(merged, ref, where=f"merge of {n} parts")
    G.assert_lse_close(merged_lse.astype(np.float32), ref_lse, where=f"merge of {n} parts")
    # the merge of the parts agrees with the single call
    d = np.abs(merged - full.astype(np.float64))
    assert d.max() <= G.MAX_ABS and d.mean() <= G.MEAN_ABS
    assert np.all(merged[4] == 0) and np.all(np.isneginf(merged_lse[4]))
    print(f"context-parallel merge of {n} parts ({layout}): max |merge - single| {d.max():.2e}")
