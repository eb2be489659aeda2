"""Seeded synthetic decode workloads for AB-Sparse (inputs only).

This module makes the inputs that both the HIP path and the CPU oracle are
fed: queries, a paged K/V cache, a shuffled page table, sequence lengths and
a per-KV-head block-size map.  It computes none of the method itself (no
centroid, score, selection or attention); the only arithmetic here shapes the
random data (outlier channels, planted needle keys, the bf16 cast).

Shapes follow the 8B-class models the AB-Sparse page evaluates on (32 query
heads, 8 KV heads, head dim 128), the page's observation that centroid
channels carry outliers (the channel-distribution figure printed after
Figure 6 of the AB-Sparse page), and the page's 16-token physical pages
grouped into 16/32/64-token logical blocks (the mapping figure after Figure 8
and the per-head block-size heatmap after Figure 3).  Every random stream is a PCG64 generator seeded with
``SeedSequence([cfg_id, layer, b, kv_head, stream])`` so that a single
(sequence, head) can be regenerated on its own.

Storage: fp32 data is ``np.float32``; bf16 data is carried as its raw 16-bit
patterns in ``np.uint16`` (numpy has no bfloat16), rounded to nearest-even.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

PAGE_SIZE = 16

# stream ids of the seed tuple
S_Q, S_K, S_V, S_OUTLIER, S_NEEDLE, S_MAP, S_PAGES = range(7)

OUTLIER_CHANNELS = 4
OUTLIER_SCALE = 10.0
NEEDLE_COS = 0.9
BLOCK_CHOICES = (16, 32, 64)
BLOCK_PROBS = (0.25, 0.25, 0.50)
# value written into cache slots past a sequence's end (never part of any
# result: a leak into a centroid or an attention output is easy to see)
PAD_SENTINEL = 512.0


@dataclass(frozen=True)
class Workload:
    cfg_id: int
    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    context: int
    dtype: str                 # "f32" or "bf16"
    token_budget: int
    needles_per_head: int
    layers: int
    fixed_block_sizes: Optional[tuple] = None

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def scaled(self, **kw) -> "Workload":
        """Same seeds and distributions, other sizes (for reduced parity cases)."""
        return dataclasses.replace(self, **kw)


PRESETS = (
    Workload(0, "tiny-gqa2-d64-2k-f32", 1, 4, 2, 64, 2048, "f32", 256, 8, 1, (16, 64)),
    Workload(1, "llama8b-32k-b1-bf16", 1, 32, 8, 128, 32768, "bf16", 2048, 16, 1),
    Workload(2, "llama8b-32k-b16-bf16", 16, 32, 8, 128, 32768, "bf16", 2048, 16, 1),
    Workload(3, "llama8b-128k-b4-bf16", 4, 32, 8, 128, 131072, "bf16", 4096, 16, 1),
    Workload(4, "qwen3-8b-64k-b8-36layer-bf16", 8, 32, 8, 128, 65536, "bf16", 2048, 16, 36),
)


def _rng(w: Workload, layer: int, b: int, h: int, stream: int) -> np.random.Generator:
    ss = np.random.SeedSequence([w.cfg_id, layer, b, h, stream])
    return np.random.Generator(np.random.PCG64(ss))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); returns the uint16 patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(x) if dtype == "bf16" else np.ascontiguousarray(x, dtype=np.float32)


def to_f32(x: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_bits_to_f32(x) if dtype == "bf16" else np.asarray(x, dtype=np.float32)


def block_sizes_for(w: Workload, layer: int) -> np.ndarray:
    """Per-KV-head block size of one layer: fixed for the tiny case, else i.i.d.
    draws from {16: 25%, 32: 25%, 64: 50%} shared by every sequence."""
    if w.fixed_block_sizes is not None:
        return np.asarray(w.fixed_block_sizes, dtype=np.int32)
    r = _rng(w, layer, 0, 0, S_MAP)
    return r.choice(np.asarray(BLOCK_CHOICES, dtype=np.int32), size=w.num_kv_heads,
                    p=BLOCK_PROBS).astype(np.int32)


@dataclass
class LayerInputs:
    workload: Workload
    layer: int
    q: np.ndarray            # [B][Hq][D] storage dtype
    k_cache: np.ndarray      # [num_pages][Hkv][16][D] storage dtype
    v_cache: np.ndarray      # same
    page_table: np.ndarray   # int32 [B][max_pages]; -1 past a sequence's pages
    seq_lens: np.ndarray     # int32 [B]
    block_size: np.ndarray   # int32 [Hkv]
    needle_pos: np.ndarray   # int64 [B][Hkv][n] token positions of planted needles
    dtype: str

    @property
    def num_pages(self) -> int:
        return int(self.k_cache.shape[0])

    @property
    def max_pages(self) -> int:
        return int(self.page_table.shape[1])


def _head_keys(w, layer, b, h, L, D, qbar, run=1):
    """Keys of one (sequence, KV head) as fp32 [L][D], plus needle positions.
    run > 1 plants the needles as runs of `run` consecutive tokens starting
    at multiples of `run` (clustered); run = 1 scatters them."""
    k = _rng(w, layer, b, h, S_K).standard_normal((L, D), dtype=np.float32)
    chans = _rng(w, layer, 0, h, S_OUTLIER).permutation(D)[:OUTLIER_CHANNELS]
    k[:, chans] *= np.float32(OUTLIER_SCALE)
    n = min(w.needles_per_head, L)
    pos = np.zeros(0, dtype=np.int64)
    if n > 0:
        r = _rng(w, layer, b, h, S_NEEDLE)
        if run > 1:
            nr = max(1, min(n // run, L // run))
            starts = r.choice(L // run, size=nr, replace=False).astype(np.int64) * run
            pos = np.sort((starts[:, None] + np.arange(run, dtype=np.int64)[None, :]).ravel())
        else:
            pos = np.sort(r.choice(L, size=n, replace=False)).astype(np.int64)
        rho = float(np.median(np.linalg.norm(k.astype(np.float64), axis=1)))
        nrm = float(np.linalg.norm(qbar))
        u = qbar / nrm if nrm > 0 else np.eye(D)[0]
        for p in pos:
            z = r.standard_normal(D)
            z -= np.dot(z, u) * u
            z /= np.linalg.norm(z)
            k[p] = (rho * (NEEDLE_COS * u + np.sqrt(1.0 - NEEDLE_COS ** 2) * z)).astype(np.float32)
    return k, pos


def make_layer(w: Workload, layer: int = 0, *, seq_lens: Optional[Sequence[int]] = None,
               block_sizes: Optional[Sequence[int]] = None, shuffle_pages: bool = True,
               needles: bool = True, extra_pages: int = 0,
               needle_runs: Optional[Sequence[int]] = None) -> LayerInputs:
    """Generate one layer's decode inputs.

    ``seq_lens`` overrides the context per sequence (ragged batches);
    ``block_sizes`` overrides the drawn map; ``shuffle_pages=False`` gives the
    identity page table; ``extra_pages`` adds unused physical pages to the pool;
    ``needle_runs`` (per KV head) plants that head's needles in aligned runs
    of that many tokens instead of scattering them (1).
    """
    B, Hq, Hkv, D, G = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.group
    lens = np.asarray(seq_lens if seq_lens is not None else [w.context] * B, dtype=np.int32)
    assert lens.shape == (B,) and (lens >= 1).all()
    bsz = (np.asarray(block_sizes, dtype=np.int32) if block_sizes is not None
           else block_sizes_for(w, layer))
    assert bsz.shape == (Hkv,)
    runs = [1] * Hkv if needle_runs is None else [int(r) for r in needle_runs]
    assert len(runs) == Hkv and min(runs) >= 1

    q32 = np.stack([_rng(w, layer, b, 0, S_Q).standard_normal((Hq, D), dtype=np.float32)
                    for b in range(B)])
    q = to_storage(q32, w.dtype)
    qf = to_f32(q, w.dtype).astype(np.float64)

    npages = (lens + PAGE_SIZE - 1) // PAGE_SIZE
    total = int(npages.sum()) + int(extra_pages)
    max_pages = int(npages.max())
    if shuffle_pages:
        perm = _rng(w, layer, 0, 0, S_PAGES).permutation(total).astype(np.int32)
    else:
        perm = np.arange(total, dtype=np.int32)
    page_table = np.full((B, max_pages), -1, dtype=np.int32)
    start = 0
    for b in range(B):
        page_table[b, :npages[b]] = perm[start:start + npages[b]]
        start += int(npages[b])

    sdt = np.uint16 if w.dtype == "bf16" else np.float32
    pad = to_storage(np.float32([PAD_SENTINEL]), w.dtype)[0]
    k_cache = np.full((total, Hkv, PAGE_SIZE, D), pad, dtype=sdt)
    v_cache = np.full((total, Hkv, PAGE_SIZE, D), pad, dtype=sdt)
    nmax = min(max(w.needles_per_head, max(runs)), int(lens.max())) if needles else 0
    needle_pos = np.full((B, Hkv, nmax), -1, dtype=np.int64)
    wn = w if needles else dataclasses.replace(w, needles_per_head=0)

    def fill(b, h):   # every (b, h) writes disjoint cache slices
        L, P = int(lens[b]), int(npages[b])
        phys = page_table[b, :P]
        qbar = qf[b, h * G:(h + 1) * G].sum(axis=0)
        k, pos = _head_keys(wn, layer, b, h, L, D, qbar, runs[h])
        needle_pos[b, h, :len(pos)] = pos
        v = _rng(w, layer, b, h, S_V).standard_normal((L, D), dtype=np.float32)
        kp = np.full((P * PAGE_SIZE, D), PAD_SENTINEL, dtype=np.float32)
        vp = np.full((P * PAGE_SIZE, D), PAD_SENTINEL, dtype=np.float32)
        kp[:L] = k
        vp[:L] = v
        k_cache[phys, h] = to_storage(kp, w.dtype).reshape(P, PAGE_SIZE, D)
        v_cache[phys, h] = to_storage(vp, w.dtype).reshape(P, PAGE_SIZE, D)

    pairs = [(b, h) for b in range(B) for h in range(Hkv)]
    if B * Hkv * int(lens.max()) * D < (1 << 22):
        for bh in pairs:
            fill(*bh)
    else:
        workers = max(1, min(8, os.cpu_count() or 1))
        with ThreadPoolExecutor(workers) as ex:
            list(ex.map(lambda bh: fill(*bh), pairs))
    return LayerInputs(w, layer, q, k_cache, v_cache, page_table, lens, bsz, needle_pos, w.dtype)


def contiguous_kv(x: LayerInputs, which: str, b: int) -> np.ndarray:
    """Un-paged [Hkv][L_b][D] fp32 view of sequence b's keys or values (a gather
    through the page table, used by tests that need the plain cache)."""
    cache = x.k_cache if which == "k" else x.v_cache
    L = int(x.seq_lens[b])
    P = (L + PAGE_SIZE - 1) // PAGE_SIZE
    pages = cache[x.page_table[b, :P]]                      # [P][Hkv][16][D]
    flat = to_f32(pages, x.dtype).transpose(1, 0, 2, 3).reshape(pages.shape[1], P * PAGE_SIZE, -1)
    return flat[:, :L]
