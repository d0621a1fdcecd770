"""Negative controls: the attention parity tolerance (max abs 2e-2, mean abs
2e-3 on fp32 output) is tight enough to see an index that is off by one, a
page table that is off by one, and set (0/1) instead of multiset semantics
for duplicated entries.  CPU only (oracle against a mistaken copy of its own
inputs)."""
import numpy as np

import oracle_pins as P
import workloads as W

MAX_TOL = 2e-2


def _run(orc, wl, pool, topk=None, page_table=None):
    return orc.sparse_attn(wl.q, pool, wl.layout,
                           wl.topk if topk is None else topk, wl.softmax_scale,
                           page_table=wl.page_table if page_table is None else page_table,
                           page_size=wl.page_size, token_seq=wl.token_seq,
                           seq_lens=wl.seq_lens)[0]


def test_wrong_index_is_visible(orc):
    wl = W.tiny_decode()
    pool = P.build_pool(orc, wl)
    ref = _run(orc, wl, pool)
    bad = wl.topk.copy()
    valid = bad >= 0
    bad[valid] = np.where(bad[valid] > 0, bad[valid] - 1, bad[valid] + 1)
    assert np.max(np.abs(_run(orc, wl, pool, topk=bad) - ref)) > 10 * MAX_TOL


def test_wrong_page_is_visible(orc):
    wl = W.tiny_decode()
    pool = P.build_pool(orc, wl)
    ref = _run(orc, wl, pool)
    pt = wl.page_table.copy()
    pt[0] = np.roll(pt[0], 1)
    assert np.max(np.abs(_run(orc, wl, pool, page_table=pt) - ref)) > 10 * MAX_TOL


def test_set_semantics_is_visible(orc):
    wl = W.small(7, T=4, H=16, K=256, layout=W.SCALED, seq_len=200, page_size=16,
                 dup_frac=0.3, neg_frac=0.0)
    pool = P.build_pool(orc, wl)
    ref = _run(orc, wl, pool)
    dedup = np.full_like(wl.topk, -1)
    for t in range(wl.T):
        u = np.unique(wl.topk[t][wl.topk[t] >= 0])
        dedup[t, :len(u)] = u
    assert np.max(np.abs(_run(orc, wl, pool, topk=dedup) - ref)) > MAX_TOL
