"""Seeded synthetic inputs for the DSA sparse-attention path.

Shared by the tests (for both the oracle and the HIP path) and by the
benchmark.  This module draws random numbers and lays out pages; it holds none
of the method's arithmetic: no FP8 encoding, no index resolution through the
page table, no softmax.  Pool bytes are produced elsewhere (by the oracle's
writer for parity inputs, by the product writer for benchmark filler).

The named workloads follow the configurations the library is measured on
(sizes and distributions in each builder's docstring).  Every draw comes from
``numpy.random.Generator(PCG64)`` children spawned from the workload's seed in
a fixed order: pool, pages, q, topk, extras.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

D = 512
RAW, SCALED, ROPE, BF16 = 0, 1, 2, 3
ROW_BYTES = {RAW: 512, SCALED: 528, ROPE: 656, BF16: 1024}
ROPE_DIM = 64            # bf16 RoPE values after the 528-byte part of a 656-byte row
POISON = 0xFF  # FP8 S.1111.111 is NaN, and 0xFFFFFFFF is an fp32 NaN


def _streams(seed: int):
    ss = np.random.SeedSequence(seed)
    pool, pages, q, topk, extras = (np.random.Generator(np.random.PCG64(c))
                                    for c in ss.spawn(5))
    return pool, pages, q, topk, extras


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 values -> bf16 bit patterns (round to nearest even), uint16."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def normal_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    return bf16_bits(rng.standard_normal(shape, dtype=np.float32))


def log_uniform_scales(rng: np.random.Generator, n: int) -> np.ndarray:
    """[n, 4] fp32 group scales 2**U(-6, 2)."""
    return np.exp2(rng.uniform(-6.0, 2.0, size=(n, 4))).astype(np.float32)


@dataclasses.dataclass
class Workload:
    name: str
    T: int
    H: int
    K: int
    layout: int
    page_size: int
    num_slots: int
    page_table: Optional[np.ndarray]  # int32 [B, max_pages], -1 = no page
    seq_lens: Optional[np.ndarray]    # int32 [B]
    token_seq: Optional[np.ndarray]   # int32 [T]; None = token t is sequence t
    topk: np.ndarray                  # int32 [T, K], -1 = padding
    q: np.ndarray                     # uint16 bf16 bits [T, H, 512] (656-byte rows: 576)
    softmax_scale: float
    kv_new: Optional[np.ndarray] = None        # uint16 bf16 bits [N, 512] (or 576)
    slot_mapping: Optional[np.ndarray] = None  # int64 [N]
    q_fp8: bool = False               # query is quantised to FP8 before attention
    seed: int = 0

    @property
    def B(self) -> int:
        return 0 if self.seq_lens is None else len(self.seq_lens)

    @property
    def row_bytes(self) -> int:
        return ROW_BYTES[self.layout]

    @property
    def rope_dim(self) -> int:
        return ROPE_DIM if self.layout == ROPE else 0

    def used_pages(self, seqs=None) -> np.ndarray:
        """Physical pages owned by the given sequences (all if None)."""
        pt = self.page_table if seqs is None else self.page_table[np.asarray(seqs)]
        p = pt[pt >= 0]
        return np.unique(p.astype(np.int64))

    def page_slots(self, pages: np.ndarray) -> np.ndarray:
        """All slots of the given physical pages, ascending."""
        ps = self.page_size
        return (np.asarray(pages, np.int64)[:, None] * ps
                + np.arange(ps, dtype=np.int64)[None, :]).reshape(-1)


def softmax_scale_512() -> float:
    return float(np.float32(1.0 / math.sqrt(D)))


def _place_pages(rng, pages_per_seq, total_pages) -> np.ndarray:
    """Random physical page placement: a seeded permutation of the pool's
    pages handed out to sequences in order.  int32 [B, max_pages], -1 pad."""
    need = int(np.sum(pages_per_seq))
    assert need <= total_pages
    perm = rng.permutation(total_pages)[:need]
    max_pages = int(np.max(pages_per_seq))
    pt = np.full((len(pages_per_seq), max_pages), -1, np.int32)
    off = 0
    for b, n in enumerate(pages_per_seq):
        pt[b, :n] = perm[off:off + n]
        off += n
    return pt


def _slots_of_positions(pt_row: np.ndarray, pos: np.ndarray, page_size: int):
    """Writer input: physical slots of logical positions of one sequence."""
    return (pt_row[pos // page_size].astype(np.int64) * page_size
            + pos % page_size)


# --------------------------------------------------------------------------
# The named workloads
# --------------------------------------------------------------------------

def tiny_decode(seed: int = 1) -> Workload:
    """1 sequence of 256 tokens in a pool of 8 pages x 64 slots (the sequence's
    4 pages are a seeded pick of the 8; the other 4 stay poisoned).  4 query
    tokens at positions 252..255, H=8, bf16 q ~ N(0,1); each top-k row is 112
    positions drawn without replacement from [0, p], then 16 entries of -1."""
    r_pool, r_pages, r_q, r_topk, r_x = _streams(seed)
    page_size, total_pages, L = 64, 8, 256
    pt = _place_pages(r_pages, [L // page_size], total_pages)
    T, H, K = 4, 8, 128
    topk = np.full((T, K), -1, np.int32)
    for t in range(T):
        p = L - T + t
        topk[t, :112] = r_topk.choice(p + 1, size=112, replace=False)
    return Workload("tiny_decode", T, H, K, RAW, page_size,
                    total_pages * page_size, pt, np.array([L], np.int32),
                    np.zeros(T, np.int32), topk, normal_bf16(r_q, (T, H, D)),
                    softmax_scale_512(), seed=seed)


def decode_batch(seed: int = 2) -> Workload:
    """64 sequences x 8192 tokens, page size 64, random physical placement in a
    2^20-slot pool (8192 of 16384 pages used).  Raw 512-byte rows, H=16, bf16 q,
    one query token per sequence (its last position).  Each top-k row: 1946
    distinct uniform positions of [0, 8192) and 102 (5% of 2048) entries of -1
    at random places; K stays 2048.  The step's writer appends each sequence's
    newest latent (position 8191)."""
    r_pool, r_pages, r_q, r_topk, r_x = _streams(seed)
    B, L, page_size, num_slots = 64, 8192, 64, 1 << 20
    pt = _place_pages(r_pages, [L // page_size] * B, num_slots // page_size)
    T, H, K, n_neg = B, 16, 2048, 102
    topk = np.empty((T, K), np.int32)
    for t in range(T):
        row = np.full(K, -1, np.int32)
        keep = r_topk.choice(K, size=K - n_neg, replace=False)
        row[keep] = r_topk.choice(L, size=K - n_neg, replace=False)
        topk[t] = row
    kv_new = normal_bf16(r_x, (B, D))
    slot_mapping = np.array([_slots_of_positions(pt[b], np.array([L - 1]),
                                                 page_size)[0]
                             for b in range(B)], np.int64)
    return Workload("decode_batch", T, H, K, RAW, page_size, num_slots, pt,
                    np.full(B, L, np.int32), None, topk,
                    normal_bf16(r_q, (T, H, D)), softmax_scale_512(),
                    kv_new, slot_mapping, seed=seed)


def rope_decode(seed: int = 6) -> Workload:
    """The decode batch's shape (64 sequences x 8192 tokens, page size 64, a
    2^20-slot pool, H=16, top-k 2048 with 5% -1) over 656-byte RoPE rows
    (group-scaled latent + 64 bf16 RoPE values) and 576-wide bf16 queries."""
    wl = decode_batch(seed)
    r_q, r_x = _streams(seed)[2], _streams(seed)[4]
    return Workload("rope_decode", wl.T, wl.H, wl.K, ROPE, wl.page_size, wl.num_slots,
                    wl.page_table, wl.seq_lens, None, wl.topk,
                    normal_bf16(r_q, (wl.T, wl.H, D + ROPE_DIM)), softmax_scale_512(),
                    normal_bf16(r_x, (wl.T, D + ROPE_DIM)), wl.slot_mapping, seed=seed)


def bf16_decode(seed: int = 7) -> Workload:
    """The decode batch's shape over 1024-byte bf16 rows (the uncompressed pool
    the FP8 rows halve)."""
    wl = decode_batch(seed)
    return Workload("bf16_decode", wl.T, wl.H, wl.K, BF16, wl.page_size, wl.num_slots,
                    wl.page_table, wl.seq_lens, None, wl.topk, wl.q, softmax_scale_512(),
                    wl.kv_new, wl.slot_mapping, seed=seed)


def scaled_decode(seed: int = 3) -> Workload:
    """128 sequences x 32768 tokens, 528-byte group-scaled rows in a 2^23-slot
    pool (half the pages used).  H=16, bf16 q.  Each top-k row: 1843 distinct
    uniform positions plus 205 (10%) repeats of entries of the same row,
    shuffled; one seed-chosen sequence has every entry -1.  Row payloads are
    N(0,1) latents and the four group scales are 2**U(-6,2) (drawn per row
    where the pool is materialised, see ``pool_content``)."""
    r_pool, r_pages, r_q, r_topk, r_x = _streams(seed)
    B, L, page_size, num_slots = 128, 32768, 64, 1 << 23
    pt = _place_pages(r_pages, [L // page_size] * B, num_slots // page_size)
    T, H, K, n_dup = B, 16, 2048, 205
    topk = np.empty((T, K), np.int32)
    for t in range(T):
        base = r_topk.choice(L, size=K - n_dup, replace=False)
        dups = base[r_topk.integers(0, K - n_dup, size=n_dup)]
        row = np.concatenate([base, dups]).astype(np.int32)
        r_topk.shuffle(row)
        topk[t] = row
    empty = int(r_x.integers(0, T))
    topk[empty] = -1
    kv_new = normal_bf16(r_x, (B, D))
    slot_mapping = np.array([_slots_of_positions(pt[b], np.array([L - 1]),
                                                 page_size)[0]
                             for b in range(B)], np.int64)
    return Workload("scaled_decode", T, H, K, SCALED, page_size, num_slots, pt,
                    np.full(B, L, np.int32), None, topk,
                    normal_bf16(r_q, (T, H, D)), softmax_scale_512(),
                    kv_new, slot_mapping, seed=seed)


def q8_prefill(seed: int = 4, prefix: int = 16384, T: int = 4096,
               H: int = 32, K: int = 2048, num_slots: int = 1 << 20) -> Workload:
    """``T`` new query tokens appended to a ``prefix``-token sequence.  The
    writer first casts the new bf16 latents to raw FP8 and scatters them into
    their slots; the query is cast to FP8 with one per-tensor scale.  Token i
    sits at position p = prefix + i and selects the local window
    {p-127 .. p} (inside the freshly written tail once i >= 127) plus
    K-128 distinct uniform positions of [0, p-128], shuffled.  Where fewer
    than K positions exist, the valid ones come first and -1 pads the row."""
    r_pool, r_pages, r_q, r_topk, r_x = _streams(seed)
    page_size = 64
    L = prefix + T
    pt = _place_pages(r_pages, [-(-L // page_size)], num_slots // page_size)
    topk = np.full((T, K), -1, np.int32)
    win = 128
    for i in range(T):
        p = prefix + i
        lo = max(0, p - win + 1)
        local = np.arange(lo, p + 1, dtype=np.int64)
        n_far = min(K - len(local), lo)
        far = r_topk.choice(lo, size=n_far, replace=False) if n_far > 0 else \
            np.empty(0, np.int64)
        row = np.concatenate([local, far]).astype(np.int32)
        r_topk.shuffle(row)
        topk[i, :len(row)] = row
    kv_new = normal_bf16(r_x, (T, D))
    pos = np.arange(prefix, L, dtype=np.int64)
    slot_mapping = _slots_of_positions(pt[0], pos, page_size)
    return Workload("q8_prefill", T, H, K, RAW, page_size, num_slots, pt,
                    np.array([L], np.int32), np.zeros(T, np.int32), topk,
                    normal_bf16(r_q, (T, H, D)), softmax_scale_512(),
                    kv_new, slot_mapping, q_fp8=True, seed=seed)


def mixed_decode(seed: int = 5) -> Workload:
    """256 sequences with context lengths log-uniform in [4096, 65536] over a
    2^24-slot raw pool (8 GiB; byte offsets beyond 4 GiB).  H=64, bf16 q.
    Each sequence draws a top-k width w from {1024, 1536, 2048}: w distinct
    uniform positions of [0, len) come first, then 2048-w entries of -1."""
    r_pool, r_pages, r_q, r_topk, r_x = _streams(seed)
    B, page_size, num_slots = 256, 64, 1 << 24
    lens = np.floor(np.exp(r_pages.uniform(math.log(4096), math.log(65536),
                                           size=B))).astype(np.int64)
    lens = np.clip(lens, 4096, 65536)
    pt = _place_pages(r_pages, [-(-int(n) // page_size) for n in lens],
                      num_slots // page_size)
    T, H, K = B, 64, 2048
    widths = r_topk.choice(np.array([1024, 1536, 2048]), size=B)
    topk = np.full((T, K), -1, np.int32)
    for t in range(T):
        w = int(widths[t])
        topk[t, :w] = r_topk.choice(int(lens[t]), size=w, replace=False)
    kv_new = normal_bf16(r_x, (B, D))
    slot_mapping = np.array([_slots_of_positions(pt[b], np.array([lens[b] - 1]),
                                                 page_size)[0]
                             for b in range(B)], np.int64)
    return Workload("mixed_decode", T, H, K, RAW, page_size, num_slots, pt,
                    lens.astype(np.int32), None, topk,
                    normal_bf16(r_q, (T, H, D)), softmax_scale_512(),
                    kv_new, slot_mapping, seed=seed)


NAMED = {
    "tiny_decode": tiny_decode,
    "decode_batch": decode_batch,
    "scaled_decode": scaled_decode,
    "q8_prefill": q8_prefill,
    "mixed_decode": mixed_decode,
    "rope_decode": rope_decode,
    "bf16_decode": bf16_decode,
}


# --------------------------------------------------------------------------
# Small workloads for parity and edge cases
# --------------------------------------------------------------------------

def small(seed: int, *, T: int = 5, H: int = 16, K: int = 256,
          layout: int = RAW, B: Optional[int] = None, seq_len: int = 300,
          page_size: int = 16, extra_pages: int = 6, neg_frac: float = 0.1,
          dup_frac: float = 0.0, physical: bool = False,
          all_masked: tuple = ()) -> Workload:
    """A small paged workload spanning several tiles and a ragged tail.

    B sequences (default: one per token) of ``seq_len`` tokens on randomly
    placed pages, ``extra_pages`` spare pages left poisoned.  Each top-k row
    holds distinct positions, ``dup_frac`` of them repeated, ``neg_frac`` of
    the entries -1 at random places.  With ``physical`` the rows hold raw
    pool slots instead of positions (no page table); the slots are those of
    the workload's own pages."""
    r_pool, r_pages, r_q, r_topk, r_x = _streams(seed)
    if B is None:
        B = T
    pages_per_seq = -(-seq_len // page_size)
    total_pages = B * pages_per_seq + extra_pages
    pt = _place_pages(r_pages, [pages_per_seq] * B, total_pages)
    token_seq = (np.arange(T) % B).astype(np.int32)
    topk = np.full((T, K), -1, np.int32)
    for t in range(T):
        n_neg = int(round(neg_frac * K))
        n_val = K - n_neg
        n_dup = int(round(dup_frac * n_val))
        n_uni = min(n_val - n_dup, seq_len)
        base = r_topk.choice(seq_len, size=n_uni, replace=False)
        dups = base[r_topk.integers(0, n_uni, size=n_val - n_uni)] \
            if n_val > n_uni else np.empty(0, np.int64)
        vals = np.concatenate([base, dups])
        if physical:
            b = token_seq[t]
            vals = _slots_of_positions(pt[b], vals.astype(np.int64), page_size)
        places = r_topk.choice(K, size=len(vals), replace=False)
        topk[t, places] = vals.astype(np.int32)
    for t in all_masked:
        topk[t] = -1
    return Workload(f"small{seed}", T, H, K, layout, page_size,
                    total_pages * page_size, None if physical else pt,
                    None if physical else np.full(B, seq_len, np.int32),
                    token_seq, topk,
                    normal_bf16(r_q, (T, H, D + (ROPE_DIM if layout == ROPE else 0))),
                    softmax_scale_512(), seed=seed)


def pool_content(seed: int, n_rows: int, layout: int):
    """Latents (uint16 bf16 bits [n_rows, 512], N(0,1)) for materialised pool
    rows, plus group scales ([n_rows, 4] fp32, 2**U(-6,2)) for the scaled
    and RoPE layouts (None for raw); RoPE layout: the latents carry 64 more
    N(0,1) bf16 columns, the RoPE values.  The caller encodes the first 512
    latent values to FP8."""
    r_pool = _streams(seed)[0]
    lat = normal_bf16(r_pool, (n_rows, D))
    sc = log_uniform_scales(r_pool, n_rows) if layout in (SCALED, ROPE) else None
    if layout == ROPE:
        lat = np.concatenate([lat, normal_bf16(r_pool, (n_rows, ROPE_DIM))], axis=1)
    return lat, sc


def random_fp8_codes(rng: np.random.Generator, shape) -> np.ndarray:
    """Uniformly random finite E4M3FN codes (the two NaN codes excluded)."""
    r = rng.integers(0, 254, size=shape, dtype=np.int32)
    r = r + (r >= 0x7F)
    return r.astype(np.uint8)
