"""The index transform on the GPU against the oracle: bit-exact slots,
per-row counts and masked-entry counts, and attention over the transformed
physical slots (no page table) against the oracle over the original
positions."""
import numpy as np
import pytest
import torch

import gpu_harness as G
import oracle_pins as P
import sparse_mla_attention_gather_amd as dsa
import workloads as W

pytestmark = pytest.mark.gpu


def run_transform(topk, num_slots, k_out, page_table=None, page_size=1,
                  token_seq=None, seq_lens=None):
    T, k_in = topk.shape
    out = torch.full((T, k_out), 12345, dtype=torch.int32, device=G.DEV)
    counts = torch.full((T,), -7, dtype=torch.int32, device=G.DEV)
    err = torch.zeros(1, dtype=torch.int32, device=G.DEV)
    num_seqs = 0 if page_table is None and seq_lens is None else (
        page_table.shape[0] if page_table is not None else len(seq_lens))
    max_pages = 0 if page_table is None else page_table.shape[1]
    d = lambda a: None if a is None else G.dev(np.ascontiguousarray(a, np.int32))
    G.check(dsa.dsa_topk_transform(d(topk), T, k_in, d(page_table), page_size, max_pages,
                                   num_seqs, d(token_seq), d(seq_lens), num_slots, out,
                                   k_out, counts, err))
    torch.cuda.synchronize()
    return G.host(out), G.host(counts), int(err.item())


def check_against_oracle(orc, topk, num_slots, k_out, **kw):
    print(f"transform case T={topk.shape[0]} k_in={topk.shape[1]} k_out={k_out} "
          f"page_size={kw.get('page_size', 1)}", flush=True)
    want, want_counts, want_err = orc.topk_transform(topk, num_slots, k_out, **kw)
    got, counts, err = run_transform(topk, num_slots, k_out, **kw)
    bad = np.nonzero(got != want)
    assert len(bad[0]) == 0, (len(bad[0]), bad[0][:4], bad[1][:4], got[bad][:4], want[bad][:4])
    assert np.array_equal(counts, want_counts)
    assert err == want_err
    return got, counts


CASES = [
    # (seed, T, k_in, k_out, page_size, pages, neg_frac, with seq_lens, with token_seq)
    (1, 3, 1, 128, 64, 4, 0.0, True, False),
    (2, 5, 100, 128, 16, 12, 0.2, True, True),
    (3, 7, 1000, 1024, 64, 20, 0.1, True, False),
    (4, 2, 2048, 2048, 1, 3000, 0.05, False, True),
    (5, 9, 3000, 4096, 32, 120, 0.3, True, True),
    (6, 1, 256, 384, 64, 8, 1.0, True, False),       # every entry padding
    (7, 33, 777, 896, 128, 10, 0.0, True, False),    # ragged tail of a pass
    (8, 2, 65536, 65536, 64, 1100, 0.1, True, False),  # the widest row
]


@pytest.mark.parametrize("case", CASES, ids=[f"t{c[0]}" for c in CASES])
def test_transform_matches_oracle(orc, case):
    seed, T, k_in, k_out, psz, pages, neg, with_len, with_ts = case
    rng = np.random.default_rng(seed)
    B = max(1, T // 2) if with_ts else T
    # shuffled physical pages, some table words -1; positions up to a bit
    # beyond the table so that every masking rule fires
    total = B * pages + 5
    pt = rng.permutation(total)[:B * pages].reshape(B, pages).astype(np.int32)
    pt[rng.random(pt.shape) < 0.05] = -1
    seq_lens = rng.integers(1, pages * psz + 1, B).astype(np.int32) if with_len else None
    token_seq = rng.integers(0, B, T).astype(np.int32) if with_ts else None
    topk = rng.integers(-2, pages * psz + psz, (T, k_in)).astype(np.int32)
    topk[rng.random((T, k_in)) < neg] = -1
    num_slots = total * psz - psz // 2          # the last page partly outside the pool
    check_against_oracle(orc, topk, num_slots, k_out, page_table=pt, page_size=psz,
                         token_seq=token_seq, seq_lens=seq_lens)


def test_transform_physical_indices(orc):
    """No page table: indices are slots, masked only when negative or beyond
    the pool; compaction as with a table."""
    rng = np.random.default_rng(8)
    topk = rng.integers(-3, 1200, (6, 500)).astype(np.int32)
    check_against_oracle(orc, topk, 1000, 512)


def test_transform_bad_sequence_id(orc):
    """A token whose sequence id is outside [0, num_seqs): every non-padding
    entry masked and counted, as in the attention."""
    pt = np.arange(8, dtype=np.int32).reshape(2, 4)
    topk = np.array([[0, 5, -1, 9], [1, 2, 3, -1], [4, -1, -1, 6]], np.int32)
    got, counts, err = run_transform(topk, 64, 128, page_table=pt, page_size=4,
                                     token_seq=np.array([0, 7, -1], np.int32))
    assert np.array_equal(got[0, :3], [0, 5, 9]) and np.all(got[0, 3:] == -1)
    assert np.all(got[1:] == -1) and np.array_equal(counts, [3, 0, 0]) and err == 5


@pytest.mark.parametrize("name", ["q8_prefill", "mixed_decode", "decode_batch"])
def test_transform_full_size(orc, name):
    """The named workloads' whole index sets, bit-exact."""
    wl = W.NAMED[name]()
    check_against_oracle(orc, wl.topk, wl.num_slots, wl.K, page_table=wl.page_table,
                         page_size=wl.page_size, token_seq=wl.token_seq,
                         seq_lens=wl.seq_lens)


@pytest.mark.parametrize("layout", [W.RAW, W.SCALED], ids=["raw", "scaled"])
def test_attention_over_transformed_slots(orc, layout):
    """Attention over the transformed physical slots (page_table NULL) agrees
    with the oracle over the original positions and page table."""
    wl = W.small(501 + layout, T=24, H=16, K=1024, layout=layout, seq_len=1500,
                 page_size=64, neg_frac=0.2, dup_frac=0.1)
    pool = P.build_pool(orc, wl)
    ref, ref_lse, _ = orc.sparse_attn(wl.q, pool, wl.layout, wl.topk, wl.softmax_scale,
                                      page_table=wl.page_table, page_size=wl.page_size,
                                      token_seq=wl.token_seq, seq_lens=wl.seq_lens)
    slots, counts = check_against_oracle(orc, wl.topk, wl.num_slots, wl.K,
                                         page_table=wl.page_table, page_size=wl.page_size,
                                         token_seq=wl.token_seq, seq_lens=wl.seq_lens)
    phys = W.Workload(**{**wl.__dict__, "topk": slots, "page_table": None,
                         "seq_lens": None, "token_seq": None})
    di = G.DevInputs(phys)
    for phase in (0, 1):
        out, lse, err = G.run_attn(di, G.dev(pool), phase=phase)
        assert err == 0
        G.assert_attn_close(out, ref, where=f"transformed slots, phase {phase}")
        G.assert_lse_close(lse, ref_lse)
