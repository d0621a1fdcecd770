"""Pins that tie the CPU oracle to facts outside itself.

Each ``pin_*`` takes an ``oracle.Oracle`` and raises AssertionError when the
oracle disagrees with: values fixed by the OCP OFP8 specification (golden
file), a brute-force nearest-code search, torch's own float8_e4m3fn routines,
a dense brute-force attention over every pool slot weighted by a count
matrix (no gather), closed forms (one-hot rows, q = 0, two entries, all
masked), or exact invariants.  ``tests/test_oracle_mutants.py`` plants
mistakes in the oracle source and checks that some pin fails for each.
"""
from __future__ import annotations

import math
import os

import numpy as np
import torch

import workloads as W

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
RAW, SCALED, ROPE, BF16 = 0, 1, 2, 3


# --------------------------------------------------------------------------
# independent helpers (torch's float8 routines, numpy)
# --------------------------------------------------------------------------

def torch_dec(b: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(b, np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def torch_enc(x: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


FINITE_CODES = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)


def brute_encode(x: np.ndarray) -> np.ndarray:
    """Nearest finite E4M3FN code by exhaustive search over the 254 finite
    codes (values from torch's decoder); ties go to the even code; anything
    beyond +-448 lands on +-448 by nearest search; NaN -> 0x7F | sign; the
    sign of zero is kept."""
    x = np.asarray(x, np.float32).reshape(-1)
    vals = torch_dec(FINITE_CODES)
    out = np.empty(x.shape, np.uint8)
    step = 4096
    for i in range(0, len(x), step):
        # every code lies in [-448, 448]; moving a value that is beyond that
        # hull to +-4096 (same side) keeps its nearest code and keeps the
        # float64 distances below exact
        with np.errstate(invalid="ignore"):
            xs = np.clip(x[i:i + step].astype(np.float64), -4096.0, 4096.0)
        dist = np.abs(xs[:, None] - vals[None, :])
        best = dist.min(axis=1, keepdims=True)
        cand = dist == best
        # among equally near codes prefer an even code, and for a zero value
        # the code with the input's sign
        even = (FINITE_CODES[None, :] & 1) == 0
        sign_ok = ((FINITE_CODES[None, :] >> 7) == np.signbit(xs)[:, None])
        score = cand * 4 + (cand & even) * 2 + (cand & sign_ok) * 1
        out[i:i + step] = FINITE_CODES[np.argmax(score, axis=1)]
    # saturation: an infinity is "beyond 448" and lands on +-448
    inf = np.isinf(x)
    out[inf] = 0x7E | (np.signbit(x[inf]).astype(np.uint8) << 7)
    nan = np.isnan(x)
    out[nan] = 0x7F | (np.signbit(x[nan]).astype(np.uint8) << 7)
    return out


def all_bf16_as_f32() -> np.ndarray:
    bits = np.arange(65536, dtype=np.uint32) << 16
    return bits.view(np.float32)


def f32_from_bf16(u16: np.ndarray) -> np.ndarray:
    return (np.asarray(u16, np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------
# FP8 decode
# --------------------------------------------------------------------------

def load_golden_codes():
    rows = []
    with open(os.path.join(GOLDEN, "ofp8_e4m3fn_codes.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            code, value = line.split()[:2]
            rows.append((int(code, 16), float(value)))
    return rows


def pin_decode_spec_values(orc):
    for code, value in load_golden_codes():
        got = orc.fp8_decode(np.array([code], np.uint8))[0]
        if math.isnan(value):
            assert math.isnan(got), (hex(code), got)
        else:
            assert got == value and math.copysign(1, got) == math.copysign(1, value), \
                (hex(code), got, value)


def pin_decode_all_codes_vs_torch(orc):
    codes = np.arange(256, dtype=np.uint8)
    got = orc.fp8_decode(codes)
    ref = torch_dec(codes)
    both_nan = np.isnan(got) & np.isnan(ref)
    assert np.all(both_nan | (got == ref)), codes[~(both_nan | (got == ref))]
    assert np.array_equal(np.signbit(got[~both_nan]), np.signbit(ref[~both_nan]))
    assert np.isnan(got).sum() == 2


def pin_decode_not_fnuz(orc):
    """E4M3FN and E4M3FNUZ disagree on these codes; the oracle must be FN."""
    codes = np.array([0x38, 0x7E, 0x80], np.uint8)
    fnuz = torch.from_numpy(codes).view(torch.float8_e4m3fnuz).to(torch.float64).numpy()
    got = orc.fp8_decode(codes)
    assert got[0] == 1.0 and fnuz[0] == 0.5
    assert got[1] == 448.0 and fnuz[1] == 224.0
    assert got[2] == 0.0 and np.signbit(got[2]) and np.isnan(fnuz[2])


# --------------------------------------------------------------------------
# FP8 encode
# --------------------------------------------------------------------------

def pin_encode_all_bf16_brute_force(orc):
    x = all_bf16_as_f32()
    got = orc.fp8_encode(x)
    ref = brute_encode(x)
    bad = np.nonzero(got != ref)[0]
    assert len(bad) == 0, [(float(x[i]), hex(got[i]), hex(ref[i])) for i in bad[:8]]


def pin_encode_midpoints(orc):
    """Every midpoint between adjacent finite codes, one fp32 ulp either side
    of it, and its negation: rounding direction and ties-to-even."""
    pos = FINITE_CODES[FINITE_CODES < 0x80]
    vals = torch_dec(pos)
    order = np.argsort(vals)
    vals, pos = vals[order], pos[order]
    xs = []
    for a, b in zip(vals[:-1], vals[1:]):
        m = np.float32((a + b) / 2)
        assert float(m) == (a + b) / 2  # exact in fp32
        xs += [m, np.nextafter(m, np.float32(0)), np.nextafter(m, np.float32(np.inf))]
    # beyond the largest code: 448 < x < 464 rounds to 448, 464 and above
    # saturate to 448 as well
    xs += [np.float32(v) for v in (448.5, 463.99, 464.0, 465.0, 480.0, 1e6, np.inf)]
    xs = np.array(xs, np.float32)
    xs = np.concatenate([xs, -xs])
    got = orc.fp8_encode(xs)
    ref = brute_encode(xs)
    bad = np.nonzero(got != ref)[0]
    assert len(bad) == 0, [(float(xs[i]), hex(got[i]), hex(ref[i])) for i in bad[:8]]


def pin_encode_random_f32(orc):
    rng = np.random.default_rng(1234)
    x = np.concatenate([
        rng.standard_normal(200_000).astype(np.float32) * np.float32(
            2.0) ** rng.integers(-14, 10, 200_000).astype(np.float32),
        rng.uniform(-470, 470, 50_000).astype(np.float32),
        rng.uniform(-2.0 ** -5, 2.0 ** -5, 50_000).astype(np.float32),
    ])
    got = orc.fp8_encode(x)
    ref = brute_encode(x)
    assert np.array_equal(got, ref)


def pin_encode_matches_torch_in_range(orc):
    """torch's cast agrees wherever it does not overflow (|x| < 464)."""
    x = all_bf16_as_f32()
    keep = np.isfinite(x) & (np.abs(x) < 464.0)
    assert np.array_equal(orc.fp8_encode(x[keep]), torch_enc(x[keep]))


def pin_encode_round_trip(orc):
    vals = torch_dec(FINITE_CODES).astype(np.float32)
    assert np.array_equal(orc.fp8_encode(vals), FINITE_CODES)


def pin_encode_special(orc):
    x = np.array([np.nan, -np.nan, np.inf, -np.inf, 0.0, -0.0, 1e-30, -1e-30],
                 np.float32)
    x[1] = -np.abs(x[1])
    got = orc.fp8_encode(x)
    assert list(got) == [0x7F, 0xFF, 0x7E, 0xFE, 0x00, 0x80, 0x00, 0x80], \
        [hex(g) for g in got]


# --------------------------------------------------------------------------
# writer
# --------------------------------------------------------------------------

def _writer_inputs(seed, n, spread=False):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, 512)).astype(np.float32)
    if spread:
        # per-group magnitudes over many binades, some all-zero groups
        mag = np.float32(2.0) ** rng.integers(-20, 12, (n, 4)).astype(np.float32)
        x = x * np.repeat(mag, 128, axis=1)
        x[0, 128:256] = 0.0
        x[1, :128] = -0.0
    return W.bf16_bits(x)


def pin_writer_raw(orc):
    kv = _writer_inputs(7, 40)
    num_slots = 64
    rng = np.random.default_rng(8)
    slots = rng.permutation(num_slots)[:40].astype(np.int64)
    slots[3] = -1           # skipped silently
    slots[5] = num_slots    # out of range: skipped and counted
    pool = np.full((num_slots, 512), 0xFF, np.uint8)
    err = orc.kv_write(kv, slots, pool, RAW)
    assert err == 1
    written = np.zeros(num_slots, bool)
    for i, s in enumerate(slots):
        if 0 <= s < num_slots:
            written[s] = True
            assert np.array_equal(pool[s], torch_enc(f32_from_bf16(kv[i])))
    assert np.all(pool[~written] == 0xFF)


def pin_writer_raw_row_stride(orc):
    """Rows taken from a wider tensor (only the first 512 columns are read)."""
    wide = _writer_inputs(9, 6)
    wide = np.concatenate([wide, np.zeros((6, 64), np.uint16)], axis=1)
    pool_a = np.zeros((6, 512), np.uint8)
    pool_b = np.zeros((6, 512), np.uint8)
    orc.kv_write(wide[:, :512], np.arange(6), pool_a, RAW)
    orc.kv_write(np.ascontiguousarray(wide[:, :512]), np.arange(6), pool_b, RAW)
    assert np.array_equal(pool_a, pool_b)


def pin_writer_scaled(orc):
    kv = _writer_inputs(11, 24, spread=True)
    x = f32_from_bf16(kv)
    pool = np.full((30, 528), 0xFF, np.uint8)
    slots = np.arange(24, dtype=np.int64) + 3
    orc.kv_write(kv, slots, pool, SCALED)
    for i in range(24):
        row = pool[slots[i]]
        scales = row[512:].view(np.float32)
        for g in range(4):
            xg = x[i, 128 * g:128 * (g + 1)]
            amax = np.max(np.abs(xg))
            want = np.float32(1.0) if amax == 0 else np.float32(amax) / np.float32(448.0)
            assert scales[g].view(np.uint32) == np.float32(want).view(np.uint32), (i, g)
            codes = row[128 * g:128 * (g + 1)]
            assert np.array_equal(codes, torch_enc(xg / want)), (i, g)
            dec = torch_dec(codes)
            if amax > 0:
                assert np.max(np.abs(dec)) == 448.0
            err = np.abs(xg.astype(np.float64) - dec * float(want))
            bound = np.maximum(2.0 ** -4 * np.abs(xg), 2.0 ** -10 * float(want))
            assert np.all(err <= bound * (1 + 1e-6)), (i, g)
    assert np.all(pool[:3] == 0xFF) and np.all(pool[27:] == 0xFF)


# --------------------------------------------------------------------------
# query quantisation
# --------------------------------------------------------------------------

def pin_q_quantize(orc):
    rng = np.random.default_rng(21)
    x = (rng.standard_normal(4 * 3 * 512) * 3).astype(np.float32)
    q = W.bf16_bits(x)
    xf = f32_from_bf16(q)
    s = orc.q_scale(q)
    want = np.float32(np.max(np.abs(xf))) / np.float32(448.0)
    assert s.view(np.uint32) == want.view(np.uint32)
    q8 = orc.q_quantize(q, s)
    assert np.array_equal(q8, torch_enc(xf / want))
    assert np.max(np.abs(torch_dec(q8))) == 448.0
    z = np.zeros(64, np.uint16)
    assert orc.q_scale(z) == 1.0
    assert np.all(orc.q_quantize(z, np.float32(1.0)) == 0)


# --------------------------------------------------------------------------
# index resolution
# --------------------------------------------------------------------------

def pin_resolve_worked_example(orc):
    """Hand-computed: page size 4, sequence 0 on physical pages [5, 2],
    sequence 1 on [7, -1], seq_lens [8, 3], a pool of 32 slots (8 pages)."""
    pt = np.array([[5, 2], [7, -1]], np.int32)
    topk = np.array([
        [0, 3, 4, 7, -1, 8, -2, 5],     # token of sequence 0
        [0, 1, 2, 3, 4, -1, 6, 2],      # token of sequence 1
    ], np.int32)
    slots, err = orc.resolve(topk, 32, page_table=pt, page_size=4,
                             token_seq=np.array([0, 1], np.int32),
                             seq_lens=np.array([8, 3], np.int32))
    want = np.array([
        [20, 23, 8, 11, -1, -1, -1, 9],
        [28, 29, 30, -1, -1, -1, -1, 30],
    ])
    assert np.array_equal(slots, want), slots
    # errors: seq0: 8 (>= len), -2; seq1: 3, 4, 6 (>= len 3)
    assert err == 5, err
    # without seq_lens the table capacity bounds sequence 1: 4..7 -> page 1 = -1
    slots, err = orc.resolve(topk, 32, page_table=pt, page_size=4,
                             token_seq=np.array([0, 1], np.int32))
    assert np.array_equal(slots[1], [28, 29, 30, 31, -1, -1, -1, 30]), slots
    assert np.array_equal(slots[0], [20, 23, 8, 11, -1, -1, -1, 9]), slots
    # physical indices (no table), pool of 10 slots
    slots, err = orc.resolve(np.array([[0, 9, 10, -1, -5]], np.int32), 10)
    assert np.array_equal(slots, [[0, 9, -1, -1, -1]]) and err == 2


def pin_resolve_page_boundaries(orc):
    """Positions 63/64 and 127/128 on non-adjacent physical pages."""
    pt = np.array([[9, 2, 14]], np.int32)
    topk = np.array([[63, 64, 127, 128, 0, 191]], np.int32)
    slots, err = orc.resolve(topk, 16 * 64, page_table=pt, page_size=64,
                             token_seq=np.zeros(1, np.int32))
    assert np.array_equal(slots, [[9 * 64 + 63, 2 * 64, 2 * 64 + 63, 14 * 64,
                                   9 * 64, 14 * 64 + 63]]) and err == 0


def pin_transform_worked_example(orc):
    """The resolution example above, compacted by hand: each row's valid
    slots in input order, then -1 to the output width; 5 masked entries."""
    pt = np.array([[5, 2], [7, -1]], np.int32)
    topk = np.array([
        [0, 3, 4, 7, -1, 8, -2, 5],
        [0, 1, 2, 3, 4, -1, 6, 2],
    ], np.int32)
    out, counts, err = orc.topk_transform(topk, 32, 128, page_table=pt, page_size=4,
                                          token_seq=np.array([0, 1], np.int32),
                                          seq_lens=np.array([8, 3], np.int32))
    assert out.shape == (2, 128)
    assert np.array_equal(out[0, :5], [20, 23, 8, 11, 9]) and np.all(out[0, 5:] == -1)
    assert np.array_equal(out[1, :4], [28, 29, 30, 30]) and np.all(out[1, 4:] == -1)
    assert np.array_equal(counts, [5, 4]) and err == 5


def pin_transform_identity_table(orc):
    """Special case: page size 1 and page_table[s][p] = p, so a slot is its
    position; the output is then numpy's boolean compaction of each row's
    non-negative positions, for widths that are and are not multiples of
    128, with padding of any length and all-padding rows."""
    rng = np.random.default_rng(5)
    for T, k_in, k_out in ((3, 1, 128), (4, 100, 128), (5, 1000, 1024), (2, 2048, 4096)):
        n_pos = 5000
        topk = rng.integers(0, n_pos, (T, k_in)).astype(np.int32)
        topk[rng.random((T, k_in)) < 0.3] = -1
        topk[0] = -1
        pt = np.tile(np.arange(n_pos, dtype=np.int32), (T, 1))
        out, counts, err = orc.topk_transform(topk, n_pos, k_out, page_table=pt, page_size=1)
        assert err == 0
        for t in range(T):
            want = topk[t][topk[t] >= 0]
            assert counts[t] == len(want)
            assert np.array_equal(out[t, :len(want)], want)
            assert np.all(out[t, len(want):] == -1)


def pin_transform_shifted_table(orc):
    """Closed form: page_table[s][p] = p + 3 with page size 64 puts position
    i at slot i + 192; positions >= seq_len, below -1, or on pages beyond
    the table are dropped and counted; -1 is dropped and not counted."""
    rng = np.random.default_rng(6)
    T, k_in, P_, pages = 6, 700, 64, 20
    pt = np.tile(np.arange(pages, dtype=np.int32) + 3, (T, 1))
    seq_lens = rng.integers(200, pages * P_ + 300, T).astype(np.int32)
    topk = rng.integers(-3, pages * P_ + 200, (T, k_in)).astype(np.int32)
    out, counts, err = orc.topk_transform(topk, (pages + 3) * P_, 768, page_table=pt,
                                          page_size=P_, seq_lens=seq_lens)
    want_err = 0
    for t in range(T):
        row = topk[t]
        ok = (row >= 0) & (row < seq_lens[t]) & (row < pages * P_)
        want = row[ok] + 3 * P_
        want_err += int(np.sum((row != -1) & ~ok))
        assert counts[t] == len(want)
        assert np.array_equal(out[t, :len(want)], want)
        assert np.all(out[t, len(want):] == -1)
    assert err == want_err


# --------------------------------------------------------------------------
# attention
# --------------------------------------------------------------------------

def build_pool(orc, wl: W.Workload, poison=True):
    """Materialise every used page of ``wl`` with the oracle's own writer
    (raw) plus drawn group scales (scaled); spare pages stay poisoned."""
    pool = np.full((wl.num_slots, wl.row_bytes), W.POISON if poison else 0,
                   np.uint8)
    if wl.page_table is not None:
        slots = wl.page_slots(wl.used_pages())
    else:
        slots = np.arange(wl.num_slots, dtype=np.int64)
    lat, sc = W.pool_content(wl.seed, len(slots), wl.layout)
    if wl.layout == RAW:
        orc.kv_write(lat, slots, pool, RAW)
    elif wl.layout == BF16:        # the latents themselves, little-endian bf16
        pool[slots] = np.ascontiguousarray(lat).view(np.uint8)
    else:
        tmp = np.zeros((len(slots), 512), np.uint8)
        orc.kv_write(lat[:, :512], np.arange(len(slots)), tmp, RAW)
        pool[slots, :512] = tmp
        pool[slots, 512:528] = sc.view(np.uint8).reshape(len(slots), 16)
        if wl.layout == ROPE:      # the RoPE values as little-endian bf16
            pool[slots, 528:656] = np.ascontiguousarray(lat[:, 512:]).view(np.uint8)
    return pool


def dequant_pool(pool, layout):
    if layout == BF16:
        return f32_from_bf16(np.ascontiguousarray(pool).view(np.uint16)).astype(np.float64)
    x = torch_dec(pool[:, :512])
    if layout in (SCALED, ROPE):
        sc = pool[:, 512:528].copy().view(np.float32).astype(np.float64)
        x = x * np.repeat(sc, 128, axis=1)
    return x


def rope_pool(pool):
    """The RoPE values of 656-byte rows, fp64 [slots, 64]."""
    return f32_from_bf16(np.ascontiguousarray(pool[:, 528:656]).view(np.uint16)).astype(np.float64)


def count_matrix(wl: W.Workload):
    """C[t, slot] = number of times token t's row names ``slot``, written out
    independently of the oracle (numpy, no shared code)."""
    C = np.zeros((wl.T, wl.num_slots))
    for t in range(wl.T):
        seq = t if wl.token_seq is None else int(wl.token_seq[t])
        for i in wl.topk[t]:
            i = int(i)
            if i < 0:
                continue
            if wl.seq_lens is not None and i >= wl.seq_lens[seq]:
                continue
            if wl.page_table is not None:
                page = i // wl.page_size
                if page >= wl.page_table.shape[1] or wl.page_table[seq, page] < 0:
                    continue
                slot = int(wl.page_table[seq, page]) * wl.page_size + i % wl.page_size
            else:
                slot = i
            if slot < wl.num_slots:
                C[t, slot] += 1
    return C


def dense_attention(qhat, X, C, scale, Xk=None):
    """Full attention over every slot, each weighted by its multiplicity.
    Keys are Xk (default X: the latent row is both key and value)."""
    T, H, _ = qhat.shape
    Xk = X if Xk is None else Xk
    out = np.zeros((T, H, 512))
    lse = np.full((T, H), -np.inf)
    for t in range(T):
        live = C[t] > 0
        if not live.any():
            continue
        Xl = X[live]
        s = float(scale) * (qhat[t] @ Xk[live].T)     # [H, n]
        M = s.max(axis=1, keepdims=True)
        w = C[t, live][None, :] * np.exp(s - M)
        L = w.sum(axis=1, keepdims=True)
        out[t] = (w @ Xl) / L
        lse[t] = (M + np.log(L))[:, 0]
    return out, lse


def _qhat(wl):
    return f32_from_bf16(wl.q).astype(np.float64)


def _run(orc, wl, pool, **kw):
    return orc.sparse_attn(wl.q, pool, wl.layout, wl.topk, wl.softmax_scale,
                           page_table=wl.page_table, page_size=wl.page_size,
                           token_seq=wl.token_seq, seq_lens=wl.seq_lens, **kw)


def _close(a, b, rtol=1e-12, atol=1e-12):
    fa, fb = np.isfinite(a), np.isfinite(b)
    assert np.array_equal(fa, fb)
    assert np.array_equal(a[~fa], b[~fb])
    assert np.allclose(a[fa], b[fb], rtol=rtol, atol=atol), \
        np.max(np.abs(a[fa] - b[fb]))


def pin_attention_dense_brute_force(orc):
    for layout, dup in ((RAW, 0.0), (SCALED, 0.2), (RAW, 0.3)):
        wl = W.small(31 + layout, T=4, H=8, K=128, layout=layout, seq_len=96,
                     page_size=16, dup_frac=dup, all_masked=(2,))
        pool = build_pool(orc, wl)
        out, lse, err = _run(orc, wl, pool)
        assert err == 0
        ref, ref_lse = dense_attention(_qhat(wl), dequant_pool(pool, layout),
                                       count_matrix(wl), wl.softmax_scale)
        _close(out, ref)
        _close(lse, ref_lse)


def pin_writer_rope(orc):
    """656-byte rows: bytes 0..527 are exactly the 528-byte writer's bytes of
    the first 512 values, bytes 528..655 the 64 RoPE values' bf16 bit
    patterns, little-endian (numpy's view of the input)."""
    rng = np.random.default_rng(71)
    n = 40
    kv = W.normal_bf16(rng, (n, 576))
    kv[3, 512:] = 0
    kv[5, :512] = 0
    slots = rng.permutation(64)[:n].astype(np.int64)
    slots[7] = -1
    rope = np.full((64, 656), 0xAB, np.uint8)
    scaled = np.full((64, 528), 0xAB, np.uint8)
    assert orc.kv_write(kv, slots, rope, ROPE) == 0
    assert orc.kv_write(np.ascontiguousarray(kv[:, :512]), slots, scaled, SCALED) == 0
    assert np.array_equal(rope[:, :528], scaled)
    ok = slots >= 0
    assert np.array_equal(rope[slots[ok], 528:], np.ascontiguousarray(kv[ok, 512:]).view(np.uint8))
    untouched = np.setdiff1d(np.arange(64), slots[ok])
    assert np.all(rope[untouched] == 0xAB)


def pin_writer_bf16(orc):
    """1024-byte rows: the writer stores the 512 bf16 values unchanged
    (numpy's byte view of the input), and touches no other slot."""
    rng = np.random.default_rng(72)
    n = 30
    kv = W.normal_bf16(rng, (n, 600))
    slots = rng.permutation(50)[:n].astype(np.int64)
    slots[4] = -1
    pool = np.full((50, 1024), 0xCD, np.uint8)
    assert orc.kv_write(kv, slots, pool, BF16) == 0
    ok = slots >= 0
    assert np.array_equal(pool[slots[ok]], np.ascontiguousarray(kv[ok, :512]).view(np.uint8))
    assert np.all(pool[np.setdiff1d(np.arange(50), slots[ok])] == 0xCD)


def pin_attention_bf16_dense_brute_force(orc):
    """1024-byte bf16 rows against dense attention over every slot."""
    for dup in (0.0, 0.3):
        wl = W.small(64, T=4, H=8, K=128, layout=BF16, seq_len=96, page_size=16,
                     dup_frac=dup, all_masked=(3,))
        pool = build_pool(orc, wl)
        out, lse, err = _run(orc, wl, pool)
        assert err == 0
        ref, ref_lse = dense_attention(_qhat(wl), dequant_pool(pool, BF16),
                                       count_matrix(wl), wl.softmax_scale)
        _close(out, ref)
        _close(lse, ref_lse)


def pin_attention_rope_dense_brute_force(orc):
    """656-byte rows against dense attention over every slot: keys are the
    dequantised latent followed by the RoPE values, values the latent only."""
    for dup in (0.0, 0.2):
        wl = W.small(61, T=4, H=8, K=128, layout=ROPE, seq_len=96, page_size=16,
                     dup_frac=dup, all_masked=(1,))
        pool = build_pool(orc, wl)
        out, lse, err = _run(orc, wl, pool)
        assert err == 0
        X = dequant_pool(pool, ROPE)
        Xk = np.concatenate([X, rope_pool(pool)], axis=1)
        ref, ref_lse = dense_attention(_qhat(wl), X, count_matrix(wl), wl.softmax_scale, Xk=Xk)
        _close(out, ref)
        _close(lse, ref_lse)


def pin_attention_rope_zero_query_part(orc):
    """A zero RoPE part of the query reduces a 656-byte row to the 528-byte
    row before it: identical results (the RoPE terms are exact zeros)."""
    wl = W.small(62, T=3, H=16, K=256, layout=ROPE, seq_len=300, page_size=16)
    q = wl.q.copy()
    q[:, :, 512:] = 0
    wl = W.Workload(**{**wl.__dict__, "q": q})
    pool = build_pool(orc, wl)
    out, lse, _ = _run(orc, wl, pool)
    wl528 = W.Workload(**{**wl.__dict__, "q": np.ascontiguousarray(q[:, :, :512]),
                          "layout": SCALED})
    out2, lse2, _ = _run(orc, wl528, np.ascontiguousarray(pool[:, :528]))
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def pin_attention_rope_only_scores(orc):
    """Closed form: a zero latent part of the query leaves s_j = scale *
    q_rope . k_rope; two live entries with RoPE parts e_0 and 2 e_0 give
    weights in the ratio exp(scale * q_rope[0] * (1 - 2))."""
    wl = W.small(63, T=1, H=8, K=128, layout=ROPE, seq_len=32, page_size=16, neg_frac=0.0)
    topk = np.full((1, 128), -1, np.int32)
    topk[0, 0], topk[0, 1] = 3, 9
    q = np.zeros_like(wl.q)
    q[0, :, 512] = W.bf16_bits(np.float32([1.5]))[0]
    wl = W.Workload(**{**wl.__dict__, "topk": topk, "q": q})
    pool = build_pool(orc, wl)
    s0, s1 = [int(wl.page_table[0, i // 16]) * 16 + i % 16 for i in (3, 9)]
    pool[[s0, s1], 528:656] = 0
    pool[s0, 528:530] = W.bf16_bits(np.float32([1.0])).view(np.uint8)
    pool[s1, 528:530] = W.bf16_bits(np.float32([2.0])).view(np.uint8)
    out, lse, err = _run(orc, wl, pool)
    X = dequant_pool(pool, ROPE)
    a = wl.softmax_scale * 1.5
    w0, w1 = 1.0, math.exp(a * (2.0 - 1.0))
    want = (w0 * X[s0] + w1 * X[s1]) / (w0 + w1)
    for h in range(8):
        _close(out[0, h], want)
        _close(np.array([lse[0, h]]), np.array([a * 1.0 + math.log(w0 + w1)]))


def pin_attention_fp8_query(orc):
    wl = W.small(41, T=3, H=8, K=128, seq_len=80, page_size=16)
    pool = build_pool(orc, wl)
    s = orc.q_scale(wl.q)
    q8 = orc.q_quantize(wl.q, s)
    out, lse, _ = orc.sparse_attn(q8, pool, RAW, wl.topk, wl.softmax_scale,
                                  q_scale=s, page_table=wl.page_table,
                                  page_size=wl.page_size, token_seq=wl.token_seq,
                                  seq_lens=wl.seq_lens)
    qhat = torch_dec(q8) * float(s)
    ref, ref_lse = dense_attention(qhat, dequant_pool(pool, RAW),
                                   count_matrix(wl), wl.softmax_scale)
    _close(out, ref)
    _close(lse, ref_lse)


def pin_attention_one_hot(orc):
    """A single valid entry returns exactly that row, lse = its score."""
    wl = W.small(51, T=3, H=8, K=128, seq_len=64, page_size=16, neg_frac=0.0)
    wl.topk[:] = -1
    wl.topk[0, 17] = 5
    wl.topk[1, 0] = 63
    wl.topk[2, 127] = 16
    pool = build_pool(orc, wl)
    out, lse, _ = _run(orc, wl, pool)
    X = dequant_pool(pool, RAW)
    for t, pos in ((0, 5), (1, 63), (2, 16)):
        seq = int(wl.token_seq[t])
        slot = int(wl.page_table[seq, pos // 16]) * 16 + pos % 16
        for h in range(wl.H):
            assert np.array_equal(out[t, h], X[slot])
            s = wl.softmax_scale * float(_qhat(wl)[t, h] @ X[slot])
            assert abs(lse[t, h] - s) <= 1e-12 * max(1.0, abs(s))


def pin_attention_zero_query(orc):
    """q = 0: every score is 0, so the output is the multiplicity-weighted
    mean of the selected rows and lse = log(count)."""
    wl = W.small(61, T=3, H=8, K=128, seq_len=64, page_size=16, dup_frac=0.3)
    wl.q[:] = 0
    pool = build_pool(orc, wl)
    out, lse, _ = _run(orc, wl, pool)
    C = count_matrix(wl)
    X = dequant_pool(pool, RAW)
    for t in range(wl.T):
        live = C[t] > 0
        mean = (C[t, live] @ X[live]) / C[t].sum()
        for h in range(wl.H):
            assert np.allclose(out[t, h], mean, rtol=1e-13, atol=1e-15)
            assert abs(lse[t, h] - math.log(C[t].sum())) < 1e-13


def pin_attention_two_entries(orc):
    """Two entries: weights are the logistic function of the score gap."""
    wl = W.small(71, T=2, H=8, K=128, seq_len=64, page_size=16)
    wl.topk[:] = -1
    wl.topk[0, 3], wl.topk[0, 99] = 10, 40
    wl.topk[1, 0], wl.topk[1, 1] = 7, 7     # a duplicated pair
    pool = build_pool(orc, wl)
    out, lse, _ = _run(orc, wl, pool)
    X = dequant_pool(pool, RAW)
    qh = _qhat(wl)

    def slot(t, pos):
        seq = int(wl.token_seq[t])
        return int(wl.page_table[seq, pos // 16]) * 16 + pos % 16

    a, b = slot(0, 10), slot(0, 40)
    for h in range(wl.H):
        sa = wl.softmax_scale * float(qh[0, h] @ X[a])
        sb = wl.softmax_scale * float(qh[0, h] @ X[b])
        wa = 1.0 / (1.0 + math.exp(sb - sa))
        assert np.allclose(out[0, h], wa * X[a] + (1 - wa) * X[b], rtol=1e-12, atol=1e-14)
        assert abs(lse[0, h] - (max(sa, sb) + math.log1p(math.exp(-abs(sa - sb))))) < 1e-12
        c = slot(1, 7)
        assert np.allclose(out[1, h], X[c], rtol=1e-15, atol=0)
        sc = wl.softmax_scale * float(qh[1, h] @ X[c])
        assert abs(lse[1, h] - (sc + math.log(2.0))) < 1e-12


def pin_attention_all_masked(orc):
    wl = W.small(81, T=3, H=8, K=128, seq_len=64, page_size=16, all_masked=(0, 2))
    pool = build_pool(orc, wl)
    out, lse, err = _run(orc, wl, pool)
    assert err == 0
    for t in (0, 2):
        assert np.all(out[t] == 0) and not np.any(np.signbit(out[t]))
        assert np.all(lse[t] == -np.inf)
    assert np.all(np.isfinite(out[1])) and np.all(np.isfinite(lse[1]))


def pin_attention_invariants(orc):
    """Order of entries and -1 placement do not matter (up to rounding)."""
    wl = W.small(91, T=3, H=8, K=128, seq_len=100, page_size=16, dup_frac=0.1)
    pool = build_pool(orc, wl)
    out, lse, _ = _run(orc, wl, pool)
    rng = np.random.default_rng(5)
    perm = wl.topk.copy()
    for t in range(wl.T):
        rng.shuffle(perm[t])
    wl2 = W.Workload(**{**wl.__dict__, "topk": perm})
    out2, lse2, _ = _run(orc, wl2, pool)
    _close(out, out2, rtol=1e-13, atol=1e-15)
    _close(lse, lse2, rtol=1e-13, atol=1e-15)
    # widen to 256 with -1 sprinkled anywhere
    wide = np.full((wl.T, 256), -1, np.int32)
    for t in range(wl.T):
        places = np.sort(rng.choice(256, 128, replace=False))
        wide[t, places] = wl.topk[t]
    wl3 = W.Workload(**{**wl.__dict__, "topk": wide, "K": 256})
    out3, lse3, _ = _run(orc, wl3, pool)
    _close(out, out3, rtol=1e-13, atol=1e-15)


def pin_attention_scaled_unit_equals_raw(orc):
    """Group scales all 1.0 reproduce the raw layout bit for bit."""
    wl = W.small(101, T=3, H=8, K=128, seq_len=64, page_size=16)
    raw = build_pool(orc, wl)
    sc = np.concatenate([raw, np.zeros((raw.shape[0], 16), np.uint8)], axis=1)
    sc[:, 512:] = np.ones((raw.shape[0], 4), np.float32).view(np.uint8)
    o1, l1, _ = _run(orc, wl, raw)
    wl2 = W.Workload(**{**wl.__dict__, "layout": SCALED})
    o2, l2, _ = _run(orc, wl2, sc)
    assert np.array_equal(o1, o2, equal_nan=True) and np.array_equal(l1, l2)


def pin_attention_power_of_two_rescale(orc):
    """Scales x 2^k with q x 2^-k: identical scores, so lse is unchanged and
    the output is exactly 2^k times the original."""
    wl = W.small(111, T=3, H=8, K=128, layout=SCALED, seq_len=64, page_size=16)
    pool = build_pool(orc, wl)
    o1, l1, _ = _run(orc, wl, pool)
    k = 3
    p2 = pool.copy()
    s = p2[:, 512:].copy().view(np.float32) * np.float32(2.0 ** k)
    p2[:, 512:] = s.view(np.uint8)
    q2 = W.bf16_bits(f32_from_bf16(wl.q) * np.float32(2.0 ** -k))
    wl2 = W.Workload(**{**wl.__dict__, "q": q2})
    o2, l2, _ = _run(orc, wl2, p2)
    assert np.array_equal(l1, l2)
    assert np.array_equal(o2, o1 * 2.0 ** k)


def pin_attention_error_count(orc):
    """-1 is padding (no error); other invalid values are masked and counted."""
    wl = W.small(121, T=2, H=8, K=128, seq_len=64, page_size=16, neg_frac=0.2)
    pool = build_pool(orc, wl)
    o1, l1, err = _run(orc, wl, pool)
    assert err == 0
    bad = wl.topk.copy()
    neg = np.nonzero(bad[0] == -1)[0]
    bad[0, neg[0]] = -7          # negative, not -1
    bad[0, neg[1]] = 64          # == seq_len
    bad[1, np.nonzero(bad[1] == -1)[0][0]] = 1 << 30   # far beyond seq_len
    wl2 = W.Workload(**{**wl.__dict__, "topk": bad})
    o2, l2, err2 = _run(orc, wl2, pool)
    assert err2 == 3, err2
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
