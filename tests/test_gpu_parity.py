"""GPU parity of the HIP path against the CPU oracle on small seeded inputs
that still span several tiles, splits and a ragged tail, plus the edge cases
(all-masked rows, -1 anywhere, duplicates, invalid indices, H not a multiple
of 16, physical indices, page size 1).  Bit-exact for the writer and the
query quantisation; attention within max abs 2e-2 / mean abs 2e-3 of the
FP64 oracle on identical dequantised inputs."""
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


def _oracle_attn(orc, wl, pool, q8=None, scale=None):
    return orc.sparse_attn(wl.q if q8 is None else q8, pool, wl.layout, wl.topk,
                           wl.softmax_scale, q_scale=scale,
                           page_table=wl.page_table, page_size=wl.page_size,
                           token_seq=wl.token_seq, seq_lens=wl.seq_lens)


# ----------------------------------------------------------------- writer

def test_writer_raw_every_bf16_pattern(orc):
    kv = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(128, 512)
    num_slots = 160
    rng = np.random.default_rng(3)
    slots = rng.permutation(num_slots)[:128].astype(np.int64)
    ref = np.full((num_slots, 512), 0xFF, np.uint8)
    assert orc.kv_write(kv, slots, ref, W.RAW) == 0
    pool = torch.full((num_slots, 512), 0xFF, dtype=torch.uint8, device=G.DEV)
    assert G.run_kv_write(kv, slots, pool, W.RAW) == 0
    got = G.host(pool)
    bad = np.nonzero(got != ref)
    assert len(bad[0]) == 0, (len(bad[0]), got[bad][:8], ref[bad][:8])


@pytest.mark.parametrize("layout", [W.RAW, W.SCALED])
def test_writer_slots_and_errors(orc, layout):
    rng = np.random.default_rng(5)
    x = rng.standard_normal((40, 512)).astype(np.float32)
    mag = np.float32(2.0) ** rng.integers(-24, 14, (40, 4)).astype(np.float32)
    x = x * np.repeat(mag, 128, axis=1)
    x[0, 128:256] = 0.0
    x[1, :128] = -0.0
    x[2, 384:] = 1e-41        # fp32 subnormal bf16 values
    kv = W.bf16_bits(x)
    R = W.ROW_BYTES[layout]
    num_slots = 50
    slots = rng.permutation(num_slots)[:40].astype(np.int64)
    slots[7] = -1
    slots[9] = num_slots
    slots[11] = 1 << 40
    ref = np.full((num_slots, R), 0xFF, np.uint8)
    ref_err = orc.kv_write(kv, slots, ref, layout)
    pool = torch.full((num_slots, R), 0xFF, dtype=torch.uint8, device=G.DEV)
    err = G.run_kv_write(kv, slots, pool, layout)
    assert err == ref_err == 2
    assert np.array_equal(G.host(pool), ref)


def test_writer_row_stride(orc):
    rng = np.random.default_rng(9)
    wide = W.bf16_bits(rng.standard_normal((6, 640)).astype(np.float32))
    ref = np.zeros((8, 528), np.uint8)
    orc.kv_write(wide[:, :512], np.arange(6), ref, W.SCALED)
    pool = torch.zeros((8, 528), dtype=torch.uint8, device=G.DEV)
    kv_d = G.dev(wide)
    sm = G.dev(np.arange(6, dtype=np.int64))
    G.check(dsa.dsa_kv_write(kv_d, 6, 640, dsa.DSA_BF16, 512, 0, sm, pool, 8,
                             W.SCALED, dsa.DSA_FP8_E4M3FN))
    torch.cuda.synchronize()
    assert np.array_equal(G.host(pool), ref)


# -------------------------------------------------------------- quantize

@pytest.mark.parametrize("n,spread", [(8, 1.0), (4096, 3.0), (3 * 16 * 512, 0.01),
                                      (1 << 21, 50.0)])
def test_quantize_bit_exact(orc, n, spread):
    rng = np.random.default_rng(n)
    q = W.bf16_bits((rng.standard_normal(n) * spread).astype(np.float32))
    q8, sc = G.run_quantize(G.dev(q))
    s_ref = orc.q_scale(q)
    assert G.host(sc)[0].view(np.uint32) == np.float32(s_ref).view(np.uint32)
    assert np.array_equal(G.host(q8), orc.q_quantize(q, s_ref))
    # given scale: only the encode runs
    q8b, _ = G.run_quantize(G.dev(q), scale_given=np.float32(0.37))
    assert np.array_equal(G.host(q8b), orc.q_quantize(q, np.float32(0.37)))


def test_quantize_zero_tensor(orc):
    q = np.zeros(1024, np.uint16)
    q[5] = 0x8000
    q8, sc = G.run_quantize(G.dev(q))
    assert G.host(sc)[0] == 1.0
    assert np.array_equal(G.host(q8), orc.q_quantize(q, np.float32(1.0)))


def _quantize_scales():
    """Divisors for the exhaustive encode test: powers of two (every quotient
    exact, so many land exactly halfway between two codes), small multiples
    of them, random log-uniform ones, and ones whose reciprocal is not a
    normal number (the division-only path)."""
    rng = np.random.default_rng(448)
    s = [1.0, 0.37, 1.0 / 448.0, 2.0 ** -7, 2.0 ** 5, 3.0 * 2.0 ** -9, 5.0 * 2.0 ** 3,
         7.0 / 448.0, 2.0 ** -125, 1e-40, 2.0 ** 125, 3e38]
    s += list(np.exp2(rng.uniform(-30, 30, 40)))
    return [np.float32(v) for v in s]


def test_quantize_every_bf16_pattern_given_scales(orc):
    """Every bf16 value (NaN, inf, subnormals, zeros of both signs included)
    divided by each divisor and encoded, bit for bit: the kernel's product by
    1/s with its exact fallback must give the codes of the IEEE quotient."""
    q = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    qd = G.dev(q)
    for sc in _quantize_scales():
        q8, _ = G.run_quantize(qd, scale_given=sc)
        ref = orc.q_quantize(q, sc)
        got = G.host(q8)
        bad = np.nonzero(got != ref)[0]
        assert len(bad) == 0, (float(sc), len(bad), q[bad][:6], got[bad][:6], ref[bad][:6])


def test_writer_scaled_every_bf16_magnitude(orc):
    """528-byte writer over groups whose largest value is set, filled with
    every finite bf16 pattern no larger than it, for several group maxima:
    codes and scales bit for bit."""
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = (pats.astype(np.uint32) << 16).view(np.float32)
    groups = []
    for amax in [1.0, 448.0, 3.3e-3, 7.5, 2.0 ** -20, 1.7e5]:
        a = np.float32(amax)
        ok = pats[np.isfinite(vals) & (np.abs(vals) <= a)]
        n = -(-len(ok) // 127) * 127
        body = np.resize(ok, n).reshape(-1, 127)
        head = np.full((body.shape[0], 1), W.bf16_bits(np.array([a], np.float32))[0], np.uint16)
        groups.append(np.concatenate([head, body], axis=1))
    g = np.concatenate(groups)
    g = np.concatenate([g, g[: (-len(g)) % 4]])
    kv = g.reshape(-1, 512)
    n = kv.shape[0]
    slots = np.arange(n, dtype=np.int64)
    ref = np.zeros((n, 528), np.uint8)
    assert orc.kv_write(kv, slots, ref, W.SCALED) == 0
    pool = torch.zeros((n, 528), dtype=torch.uint8, device=G.DEV)
    assert G.run_kv_write(kv, slots, pool, W.SCALED) == 0
    got = G.host(pool)
    bad = np.nonzero(got != ref)
    assert len(bad[0]) == 0, (len(bad[0]), bad[0][:4], bad[1][:4])


# ------------------------------------------------------------- attention

def test_fp8_decode_exact_one_hot(orc):
    """One-hot rows return the row itself, exactly, for every finite code."""
    codes = P.FINITE_CODES
    rng = np.random.default_rng(11)
    rows = np.stack([np.resize(rng.permutation(codes), 512) for _ in range(6)])
    for layout in (W.RAW, W.SCALED):
        if layout == W.RAW:
            pool = rows
        else:
            sc = np.float32(2.0) ** rng.integers(-6, 3, (6, 4)).astype(np.float32)
            pool = np.concatenate([rows, sc.view(np.uint8).reshape(6, 16)], axis=1)
        T = 6
        topk = np.full((T, 128), -1, np.int32)
        for t in range(T):
            topk[t, rng.integers(0, 128)] = t
        wl = W.Workload("onehot", T, 8, 128, layout, 1, 6, None, None, None, topk,
                        W.normal_bf16(rng, (T, 8, 512)), W.softmax_scale_512())
        ref, ref_lse, _ = _oracle_attn(orc, wl, pool)
        di = G.DevInputs(wl)
        for phase in (0, 1):
            for od in (dsa.DSA_FP32, dsa.DSA_BF16):
                out, lse, err = G.run_attn(di, G.dev(pool), phase=phase, out_dtype=od)
                assert err == 0
                assert np.array_equal(out, ref.astype(np.float32)), (layout, phase, od)
                G.assert_lse_close(lse, ref_lse)


SMALL = [
    dict(seed=201, T=5, H=16, K=256, layout=W.RAW),
    dict(seed=202, T=3, H=8, K=128, layout=W.RAW, neg_frac=0.3),
    dict(seed=203, T=4, H=32, K=384, layout=W.SCALED, dup_frac=0.2),
    dict(seed=204, T=3, H=64, K=256, layout=W.RAW, all_masked=(1,)),
    dict(seed=205, T=6, H=24, K=512, layout=W.SCALED, physical=True),
    dict(seed=206, T=3, H=16, K=1024, layout=W.RAW, seq_len=2000, page_size=64),
    dict(seed=207, T=7, H=5, K=128, layout=W.RAW, page_size=1),
    dict(seed=208, T=2, H=16, K=2048, layout=W.SCALED, seq_len=3000, page_size=64,
         dup_frac=0.1, neg_frac=0.05),
    # enough tokens that decode splits the list into several multi-tile
    # pieces (more tiles per piece than tile buffers, a shorter last piece)
    dict(seed=209, T=48, H=16, K=1664, layout=W.RAW, seq_len=2500, page_size=64),
    dict(seed=210, T=40, H=32, K=1664, layout=W.SCALED, seq_len=2000, page_size=64,
         neg_frac=0.05),
    dict(seed=211, T=24, H=64, K=896, layout=W.RAW, seq_len=1200, page_size=32),
]


@pytest.mark.parametrize("cfg", SMALL, ids=[f"s{c['seed']}" for c in SMALL])
@pytest.mark.parametrize("phase", [0, 1], ids=["decode", "prefill"])
@pytest.mark.parametrize("qfp8", [False, True], ids=["qbf16", "qfp8"])
@pytest.mark.parametrize("od", [dsa.DSA_FP32, dsa.DSA_BF16], ids=["f32", "bf16"])
def test_attention_small(orc, cfg, phase, qfp8, od):
    wl = W.small(**cfg)
    pool = P.build_pool(orc, wl)
    di = G.DevInputs(wl)
    pool_d = G.dev(pool)
    if qfp8:
        q8_d, sc_d = G.run_quantize(di.q)
        s_ref = orc.q_scale(wl.q)
        q8_ref = orc.q_quantize(wl.q, s_ref)
        assert np.array_equal(G.host(q8_d), q8_ref)
        assert G.host(sc_d)[0] == s_ref
        ref, ref_lse, ref_err = _oracle_attn(orc, wl, pool, q8_ref, s_ref)
        out, lse, err = G.run_attn(di, pool_d, phase=phase, out_dtype=od,
                                   q=q8_d, q_scale=sc_d)
    else:
        ref, ref_lse, ref_err = _oracle_attn(orc, wl, pool)
        out, lse, err = G.run_attn(di, pool_d, phase=phase, out_dtype=od)
    assert err == ref_err
    G.assert_attn_close(out, ref, od, where=str(cfg))
    G.assert_lse_close(lse, ref_lse, where=str(cfg))
    for t in cfg.get("all_masked", ()):
        assert np.all(out[t] == 0) and np.all(lse[t] == -np.inf)


# FP8 query over raw rows with more than 16 heads runs the eight-wavefront
# kernel (32-head blocks): a prefill list of several 2048-entry splits, a
# partly filled second head block, a token count that is not a multiple of 8,
# repeated and padded entries, a token with no valid entry, page size 1.
Q8_BLOCKS = [
    dict(seed=221, T=9, H=32, K=2560, layout=W.RAW, seq_len=4000, page_size=64,
         dup_frac=0.1, neg_frac=0.05, all_masked=(4,)),
    dict(seed=222, T=5, H=40, K=1152, layout=W.RAW, seq_len=1500, page_size=32),
    dict(seed=223, T=3, H=32, K=128, layout=W.RAW, seq_len=200, page_size=1, neg_frac=0.4),
]


@pytest.mark.parametrize("cfg", Q8_BLOCKS, ids=[f"s{c['seed']}" for c in Q8_BLOCKS])
@pytest.mark.parametrize("phase", [0, 1], ids=["decode", "prefill"])
@pytest.mark.parametrize("od", [dsa.DSA_FP32, dsa.DSA_BF16], ids=["f32", "bf16"])
def test_fp8_query_32_head_blocks(orc, cfg, phase, od):
    wl = W.small(**cfg)
    pool = P.build_pool(orc, wl)
    di = G.DevInputs(wl)
    q8_d, sc_d = G.run_quantize(di.q)
    s_ref = orc.q_scale(wl.q)
    q8_ref = orc.q_quantize(wl.q, s_ref)
    assert np.array_equal(G.host(q8_d), q8_ref)
    ref, ref_lse, ref_err = _oracle_attn(orc, wl, pool, q8_ref, s_ref)
    out, lse, err = G.run_attn(di, G.dev(pool), phase=phase, out_dtype=od, q=q8_d, q_scale=sc_d)
    assert err == ref_err
    G.assert_attn_close(out, ref, od, where=str(cfg))
    G.assert_lse_close(lse, ref_lse, where=str(cfg))
    for t in cfg.get("all_masked", ()):
        assert np.all(out[t] == 0) and np.all(lse[t] == -np.inf)


# The FP8-query prefill over raw rows runs persistent workgroups (one per
# compute unit), each taking several (token, head block, split) units in
# turn and starting the next one (its entries resolved, its first tiles
# copied) while the current one ends.  Tokens cycle over 5 sequences, so a
# workgroup's consecutive units read different page-table rows; rows are
# ragged (1 to 4 tiles, some empty); page-table rows of 63 pages (page size
# 16, short enough for the first unit to stage in LDS) and of 2000 pages
# (page size 1).
@pytest.mark.parametrize("page_size,seq_len", [(16, 1000), (1, 2000)], ids=["short_pt", "long_pt"])
def test_q8_prefill_persistent_units(orc, page_size, seq_len):
    T, H, K = 800, 32, 256
    wl = W.small(261 + page_size, T=T, H=H, K=K, layout=W.RAW, B=5, seq_len=seq_len,
                 page_size=page_size, neg_frac=0.0)
    widths = [0, 1, 63, 64, 65, 128, 129, 200, 256]
    topk = wl.topk.copy()
    for t in range(T):
        topk[t, widths[t % len(widths)]:] = -1
    wl = W.Workload(**{**wl.__dict__, "topk": topk})
    print(f"case persistent prefill: T={T} H={H} K={K} page_size={page_size} "
          f"pages={wl.page_table.shape[1]}", flush=True)
    pool = P.build_pool(orc, wl)
    di = G.DevInputs(wl)
    q8_d, sc_d = G.run_quantize(di.q)
    s_ref = orc.q_scale(wl.q)
    q8_ref = orc.q_quantize(wl.q, s_ref)
    assert np.array_equal(G.host(q8_d), q8_ref)
    ref, ref_lse, ref_err = _oracle_attn(orc, wl, pool, q8_ref, s_ref)
    out, lse, err = G.run_attn(di, G.dev(pool), phase=1, q=q8_d, q_scale=sc_d)
    assert err == ref_err == 0
    G.assert_attn_close(out, ref, where=f"persistent prefill, page size {page_size}")
    G.assert_lse_close(lse, ref_lse)
    for t in range(T):
        if widths[t % len(widths)] == 0:
            assert np.all(out[t] == 0) and np.all(lse[t] == -np.inf)


def test_q8_prefill_persistent_splits(orc):
    """Persistent FP8-query prefill units of a top-k list longer than one
    split (2304 entries: two splits per token, their partial states merged
    afterwards), several units per workgroup, ragged rows up to the full
    width."""
    T, H, K = 400, 32, 2304
    wl = W.small(264, T=T, H=H, K=K, layout=W.RAW, B=3, seq_len=3000, page_size=16,
                 neg_frac=0.0)
    widths = [0, 64, 700, 1200, 2100, 2304]
    topk = wl.topk.copy()
    for t in range(T):
        topk[t, widths[t % len(widths)]:] = -1
    wl = W.Workload(**{**wl.__dict__, "topk": topk})
    print(f"case persistent prefill with splits: T={T} H={H} K={K}", flush=True)
    pool = P.build_pool(orc, wl)
    di = G.DevInputs(wl)
    q8_d, sc_d = G.run_quantize(di.q)
    s_ref = orc.q_scale(wl.q)
    q8_ref = orc.q_quantize(wl.q, s_ref)
    ref, ref_lse, ref_err = _oracle_attn(orc, wl, pool, q8_ref, s_ref)
    out, lse, err = G.run_attn(di, G.dev(pool), phase=1, q=q8_d, q_scale=sc_d)
    assert err == ref_err == 0
    G.assert_attn_close(out, ref, where="persistent prefill, two splits")
    G.assert_lse_close(lse, ref_lse)
    for t in range(T):
        if widths[t % len(widths)] == 0:
            assert np.all(out[t] == 0) and np.all(lse[t] == -np.inf)


def test_q8_prefill_persistent_bad_sequence():
    """Persistent FP8-query prefill units whose token has a sequence id
    outside [0, num_seqs) (a workgroup's first and later units) read
    nothing: output 0, lse -inf, every non -1 entry counted."""
    T, H, K = 800, 32, 128
    wl = W.small(265, T=T, H=H, K=K, seq_len=100, page_size=16, B=3)
    ts = wl.token_seq.copy()
    bad = [3, 259, 515, 771]
    ts[bad] = [7, -1, 3, 1 << 20]
    wl = W.Workload(**{**wl.__dict__, "token_seq": ts})
    pool = np.zeros((wl.num_slots, 512), np.uint8)
    di = G.DevInputs(wl)
    q8_d, sc_d = G.run_quantize(di.q)
    out, lse, err = G.run_attn(di, G.dev(pool), phase=1, q=q8_d, q_scale=sc_d)
    for t in bad:
        assert np.all(out[t] == 0) and np.all(lse[t] == -np.inf), t
    assert err == int(np.sum(wl.topk[bad] != -1))


@pytest.mark.parametrize("H", [16, 32])
@pytest.mark.parametrize("layout", [W.RAW, W.SCALED, W.ROPE, W.BF16],
                         ids=["raw", "scaled", "rope", "bf16"])
@pytest.mark.parametrize("phase", [0, 1], ids=["decode", "prefill"])
def test_trailing_masked_entries(orc, layout, phase, H):
    """Rows whose valid entries end early (every later entry -1, as ragged
    widths padded to the row width): widths 0, 1, 63, 64, 65, mid-list and
    full, across several multi-tile splits.  The tiles after a split's last
    valid entry are skipped, which must not change any result."""
    widths = [0, 1, 63, 64, 65, 700, 1023, 1024, 1500, 1664]
    T = 6 * len(widths)
    wl = W.small(301 + layout, T=T, H=H, K=1664, layout=layout, seq_len=2500,
                 page_size=64, neg_frac=0.0)
    topk = wl.topk.copy()
    for t in range(T):
        topk[t, widths[t % len(widths)]:] = -1
    wl = W.Workload(**{**wl.__dict__, "topk": topk})
    pool = P.build_pool(orc, wl)
    di = G.DevInputs(wl)
    ref, ref_lse, ref_err = _oracle_attn(orc, wl, pool)
    out, lse, err = G.run_attn(di, G.dev(pool), phase=phase)
    assert err == ref_err == 0
    G.assert_attn_close(out, ref, where=f"trailing -1, layout {layout}, phase {phase}")
    G.assert_lse_close(lse, ref_lse)
    for t in range(T):
        if widths[t % len(widths)] == 0:
            assert np.all(out[t] == 0) and np.all(lse[t] == -np.inf)


@pytest.mark.parametrize("H", [16, 64])
@pytest.mark.parametrize("layout", [W.RAW, W.SCALED], ids=["raw", "scaled"])
def test_decode_more_units_than_cus(orc, layout, H):
    """Decode with more (token, head block) units than compute units (so
    workgroups run in several rounds, each split holding a whole row) and
    ragged widths (every later entry -1), tokens of equal width spread over
    the batch and a few rows empty."""
    T, K = 300, 512
    rng = np.random.default_rng(4000 + 10 * layout + H)
    widths = rng.choice([0, 1, 63, 64, 65, 200, 383, 384, 511, 512], size=T)
    wl = W.small(401 + layout, T=T, H=H, K=K, layout=layout, seq_len=700,
                 page_size=64, neg_frac=0.0)
    topk = wl.topk.copy()
    for t in range(T):
        topk[t, widths[t]:] = -1
    wl = W.Workload(**{**wl.__dict__, "topk": topk})
    pool = P.build_pool(orc, wl)
    di = G.DevInputs(wl)
    ref, ref_lse, ref_err = _oracle_attn(orc, wl, pool)
    out, lse, err = G.run_attn(di, G.dev(pool), phase=0)
    assert err == ref_err == 0
    G.assert_attn_close(out, ref, where=f"{T} tokens, H {H}, layout {layout}")
    G.assert_lse_close(lse, ref_lse)
    for t in np.nonzero(widths == 0)[0]:
        assert np.all(out[t] == 0) and np.all(lse[t] == -np.inf)


BF16_SMALL = [
    dict(seed=231, T=5, H=16, K=256, layout=W.BF16),
    dict(seed=232, T=3, H=8, K=384, layout=W.BF16, dup_frac=0.2, neg_frac=0.3),
    dict(seed=233, T=40, H=32, K=1664, layout=W.BF16, seq_len=2000, page_size=64),
    dict(seed=234, T=4, H=16, K=1024, layout=W.BF16, seq_len=1500, page_size=64,
         physical=True, all_masked=(1,)),
]


@pytest.mark.parametrize("cfg", BF16_SMALL, ids=[f"s{c['seed']}" for c in BF16_SMALL])
@pytest.mark.parametrize("phase", [0, 1], ids=["decode", "prefill"])
@pytest.mark.parametrize("od", [dsa.DSA_FP32, dsa.DSA_BF16], ids=["f32", "bf16"])
def test_attention_bf16_rows_small(orc, cfg, phase, od):
    """1024-byte bf16 rows (no FP8 anywhere) against the oracle."""
    wl = W.small(**cfg)
    pool = P.build_pool(orc, wl)
    ref, ref_lse, ref_err = _oracle_attn(orc, wl, pool)
    out, lse, err = G.run_attn(G.DevInputs(wl), G.dev(pool), phase=phase, out_dtype=od)
    assert err == ref_err
    G.assert_attn_close(out, ref, od, where=str(cfg))
    G.assert_lse_close(lse, ref_lse, where=str(cfg))
    for t in cfg.get("all_masked", ()):
        assert np.all(out[t] == 0) and np.all(lse[t] == -np.inf)


def test_writer_bf16_rows(orc):
    """The writer on 1024-byte rows stores the bf16 values unchanged."""
    rng = np.random.default_rng(18)
    n, stride = 200, 528
    kv = W.normal_bf16(rng, (n, stride))
    slots = rng.permutation(256)[:n].astype(np.int64)
    slots[::13] = -1
    ref = np.full((256, 1024), 0x3C, np.uint8)
    assert orc.kv_write(kv, slots, ref, W.BF16) == 0
    pool = torch.full((256, 1024), 0x3C, dtype=torch.uint8, device=G.DEV)
    assert G.run_kv_write(kv, slots, pool, W.BF16) == 0
    assert np.array_equal(G.host(pool), ref)


ROPE_SMALL = [
    dict(seed=221, T=5, H=16, K=256, layout=W.ROPE),
    dict(seed=222, T=3, H=8, K=384, layout=W.ROPE, dup_frac=0.2, neg_frac=0.3),
    dict(seed=223, T=40, H=32, K=1664, layout=W.ROPE, seq_len=2000, page_size=64),
    dict(seed=224, T=4, H=16, K=1024, layout=W.ROPE, seq_len=1500, page_size=64,
         physical=True, all_masked=(2,)),
]


@pytest.mark.parametrize("cfg", ROPE_SMALL, ids=[f"s{c['seed']}" for c in ROPE_SMALL])
@pytest.mark.parametrize("phase", [0, 1], ids=["decode", "prefill"])
@pytest.mark.parametrize("od", [dsa.DSA_FP32, dsa.DSA_BF16], ids=["f32", "bf16"])
def test_attention_rope_small(orc, cfg, phase, od):
    """656-byte RoPE rows (bf16 query of 512 + 64): the writer's bytes and
    the attention against the oracle."""
    wl = W.small(**cfg)
    pool = P.build_pool(orc, wl)
    ref, ref_lse, ref_err = _oracle_attn(orc, wl, pool)
    out, lse, err = G.run_attn(G.DevInputs(wl), G.dev(pool), phase=phase, out_dtype=od)
    assert err == ref_err
    G.assert_attn_close(out, ref, od, where=str(cfg))
    G.assert_lse_close(lse, ref_lse, where=str(cfg))
    for t in cfg.get("all_masked", ()):
        assert np.all(out[t] == 0) and np.all(lse[t] == -np.inf)


def test_writer_rope_rows(orc):
    """The writer on 656-byte rows, bit for bit: latent as the scaled rows,
    then the 64 RoPE values; rows read with a stride wider than 576."""
    rng = np.random.default_rng(17)
    n, stride = 300, 640
    kv = W.normal_bf16(rng, (n, stride))
    kv[:7] = W.bf16_bits(np.float32(rng.standard_normal((7, stride)) * 1e4))
    kv[9, :512] = 0
    slots = rng.permutation(400)[:n].astype(np.int64)
    slots[::17] = -1
    ref = np.full((400, 656), 0x5A, np.uint8)
    assert orc.kv_write(kv, slots, ref, W.ROPE) == 0
    pool = torch.full((400, 656), 0x5A, dtype=torch.uint8, device=G.DEV)
    assert G.run_kv_write(kv, slots, pool, W.ROPE) == 0
    got = G.host(pool)
    bad = np.nonzero(got != ref)
    assert len(bad[0]) == 0, (len(bad[0]), bad[0][:4], bad[1][:4])


@pytest.mark.parametrize("phase", [0, 1], ids=["decode", "prefill"])
@pytest.mark.parametrize("layout", [W.RAW, W.SCALED], ids=["raw", "scaled"])
def test_attention_most_heads(orc, layout, phase):
    """H = 128, the most heads the C ABI accepts (raw: four 32-head
    blocks; 528-byte rows: eight 16-head blocks)."""
    wl = W.small(241 + layout, T=2, H=128, K=256, layout=layout, seq_len=400)
    pool = P.build_pool(orc, wl)
    ref, ref_lse, ref_err = _oracle_attn(orc, wl, pool)
    out, lse, err = G.run_attn(G.DevInputs(wl), G.dev(pool), phase=phase)
    assert err == ref_err
    G.assert_attn_close(out, ref, where=f"H=128 layout {layout}")
    G.assert_lse_close(lse, ref_lse)


@pytest.mark.parametrize("phase", [0, 1], ids=["decode", "prefill"])
def test_attention_widest_topk(orc, phase):
    """K = 65536, the widest top-k list: 32 splits of 2048 entries merged in
    chunks of 8; page size 16 gives a page-table row (4375 pages) too long to
    stage in LDS, so the indices resolve through direct page-table loads."""
    wl = W.small(251, T=2, H=16, K=65536, layout=W.RAW, seq_len=70000, page_size=16,
                 neg_frac=0.02)
    print(f"case widest top-k: T={wl.T} H={wl.H} K={wl.K} pages={wl.page_table.shape[1]}",
          flush=True)
    pool = P.build_pool(orc, wl)
    ref, ref_lse, ref_err = _oracle_attn(orc, wl, pool)
    out, lse, err = G.run_attn(G.DevInputs(wl), G.dev(pool), phase=phase)
    assert err == ref_err
    G.assert_attn_close(out, ref, where="K=65536")
    G.assert_lse_close(lse, ref_lse)


def test_invalid_indices_are_masked_and_counted(orc):
    wl = W.small(301, T=4, H=16, K=256, neg_frac=0.25, seq_len=120)
    bad = wl.topk.copy()
    for t in range(wl.T):
        neg = np.nonzero(bad[t] == -1)[0]
        bad[t, neg[0]] = -5                  # negative, not -1
        bad[t, neg[1]] = 120                 # == seq_len
        bad[t, neg[2]] = 1 << 30             # far out
    wl = W.Workload(**{**wl.__dict__, "topk": bad})
    pool = P.build_pool(orc, wl)
    ref, ref_lse, ref_err = _oracle_attn(orc, wl, pool)
    assert ref_err == 12
    for phase in (0, 1):
        out, lse, err = G.run_attn(G.DevInputs(wl), G.dev(pool), phase=phase)
        assert err == ref_err
        G.assert_attn_close(out, ref)


def test_bad_page_table_entries_are_masked(orc):
    wl = W.small(302, T=3, H=16, K=256, seq_len=200, page_size=16)
    pt = wl.page_table.copy()
    pt[1, 3] = -1                            # a hole in sequence 1's table
    wl = W.Workload(**{**wl.__dict__, "page_table": pt})
    pool = P.build_pool(orc, wl)
    ref, ref_lse, ref_err = _oracle_attn(orc, wl, pool)
    assert ref_err > 0
    out, lse, err = G.run_attn(G.DevInputs(wl), G.dev(pool), phase=0)
    assert err == ref_err
    G.assert_attn_close(out, ref)


def test_out_of_range_sequence_id():
    """A token whose sequence id is outside [0, num_seqs) reads nothing: its
    output is 0, lse -inf, and every non -1 entry is counted."""
    wl = W.small(303, T=3, H=16, K=128, seq_len=100, page_size=16, B=3)
    ts = wl.token_seq.copy()
    ts[2] = 7
    wl = W.Workload(**{**wl.__dict__, "token_seq": ts})
    pool = np.zeros((wl.num_slots, 512), np.uint8)
    out, lse, err = G.run_attn(G.DevInputs(wl), G.dev(pool), phase=1)
    assert np.all(out[2] == 0) and np.all(lse[2] == -np.inf)
    assert err == int(np.sum(wl.topk[2] != -1))


@pytest.mark.parametrize("kind", ["decode", "prefill", "q8_prefill_persistent"])
def test_negative_sequence_length(kind):
    """A sequence whose length is negative holds no valid position: every
    non -1 entry of its tokens is masked and counted, output 0, lse -inf.
    Covers the 16-head kernel (decode, prefill) and the persistent FP8-query
    prefill (tokens of that sequence in a workgroup's first and later
    units)."""
    H, T = (32, 800) if kind == "q8_prefill_persistent" else (16, 9)
    wl = W.small(304, T=T, H=H, K=128, seq_len=100, page_size=16, B=3)
    sl = wl.seq_lens.copy()
    sl[1] = -5
    wl = W.Workload(**{**wl.__dict__, "seq_lens": sl})
    pool = np.zeros((wl.num_slots, 512), np.uint8)
    di = G.DevInputs(wl)
    kw = {}
    if kind == "q8_prefill_persistent":
        q8_d, sc_d = G.run_quantize(di.q)
        kw = dict(q=q8_d, q_scale=sc_d)
    out, lse, err = G.run_attn(di, G.dev(pool), phase=0 if kind == "decode" else 1, **kw)
    bad = np.nonzero(wl.token_seq == 1)[0]
    for t in bad:
        assert np.all(out[t] == 0) and np.all(lse[t] == -np.inf), t
    assert err == int(np.sum(wl.topk[bad] != -1))


@pytest.mark.parametrize("prefix,T,K", [(200, 300, 256), (0, 260, 256)])
def test_prefill_pipeline_live_tail(orc, prefix, T, K):
    """Writer -> query quantisation -> prefill, in stream order: the top-k
    lists reach into rows the writer has just appended; short histories are
    padded with -1."""
    wl = W.q8_prefill(seed=44, prefix=prefix, T=T, H=16, K=K, num_slots=1 << 14)
    # pool: prefix rows materialised by the oracle's writer, tail poisoned
    pool = np.full((wl.num_slots, 512), 0xFF, np.uint8)
    if prefix:
        lat, _ = W.pool_content(wl.seed, prefix, W.RAW)
        pos = np.arange(prefix, dtype=np.int64)
        pre_slots = wl.page_table[0][pos // 64].astype(np.int64) * 64 + pos % 64
        orc.kv_write(lat, pre_slots, pool, W.RAW)
    pool_d = G.dev(pool)
    ref_pool = pool.copy()
    orc.kv_write(wl.kv_new, wl.slot_mapping, ref_pool, W.RAW)
    assert G.run_kv_write(wl.kv_new, wl.slot_mapping, pool_d, W.RAW) == 0
    assert np.array_equal(G.host(pool_d), ref_pool)
    di = G.DevInputs(wl)
    q8_d, sc_d = G.run_quantize(di.q)
    s_ref = orc.q_scale(wl.q)
    q8_ref = orc.q_quantize(wl.q, s_ref)
    assert np.array_equal(G.host(q8_d), q8_ref)
    ref, ref_lse, _ = _oracle_attn(orc, wl, ref_pool, q8_ref, s_ref)
    out, lse, err = G.run_attn(di, pool_d, phase=1, q=q8_d, q_scale=sc_d)
    assert err == 0
    G.assert_attn_close(out, ref)
    G.assert_lse_close(lse, ref_lse)


def test_graph_replay_with_changing_inputs(orc):
    """A captured decode call replayed after its indices, queries and pool
    scales were changed in place matches the oracle each time."""
    wl = W.small(401, T=4, H=16, K=512, layout=W.SCALED, seq_len=400, page_size=16)
    pool = P.build_pool(orc, wl)
    di = G.DevInputs(wl)
    pool_d = G.dev(pool)
    T, H, K = wl.T, wl.H, wl.K
    out = torch.empty((T, H, 512), dtype=torch.float32, device=G.DEV)
    lse = torch.empty((T, H), dtype=torch.float32, device=G.DEV)
    wsb = dsa.dsa_attn_workspace_bytes(T, H, K, 0)
    ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=G.DEV)

    def call():
        G.check(dsa.dsa_sparse_attn_decode(
            di.q, dsa.DSA_BF16, None, T, H, 512, 0, pool_d, pool_d.shape[0],
            wl.layout, dsa.DSA_FP8_E4M3FN, di.topk, K, di.page_table,
            wl.page_size, di.max_pages, di.num_seqs, di.token_seq, di.seq_lens,
            wl.softmax_scale, out, dsa.DSA_FP32, lse, ws, wsb, None))

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()                                # warm-up outside capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    rng = np.random.default_rng(77)
    for it in range(3):
        # new indices, queries and group scales, written into the same buffers
        w2 = W.small(402 + it, T=4, H=16, K=512, layout=W.SCALED, seq_len=400,
                     page_size=16)
        new_topk = w2.topk
        new_q = w2.q
        new_pool = pool.copy()
        sc = new_pool[:, 512:].copy().view(np.float32)
        sc *= np.float32(2.0) ** rng.integers(-2, 3, sc.shape).astype(np.float32)
        new_pool[:, 512:] = sc.view(np.uint8)
        di.topk.copy_(torch.from_numpy(new_topk))
        di.q.copy_(torch.from_numpy(new_q.view(np.int16)))
        pool_d.copy_(torch.from_numpy(new_pool))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        wl2 = W.Workload(**{**wl.__dict__, "topk": new_topk, "q": new_q})
        ref, ref_lse, _ = _oracle_attn(orc, wl2, new_pool)
        G.assert_attn_close(G.host(out), ref, where=f"replay {it}")
        G.assert_lse_close(G.host(lse), ref_lse)
        # eager work between replays
        _ = (out.sum() + 1).item()
