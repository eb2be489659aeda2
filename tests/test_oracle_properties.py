"""Property checks of the CPU oracle over random small shapes (hypothesis):
partial last blocks, budgets that are not multiples of the block size,
K >= N, constant channels and tied scores.  Each property is stated from the
definitions (AB-Sparse page, Figure 1's stages; Figure 8's INT4 centroids;
the page-mapping figure after Figure 8), not from the oracle's code."""
import math

import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

from block_sparse_attention_abs_amd import workload as W

SETTINGS = settings(max_examples=30, deadline=None, suppress_health_check=[HealthCheck.function_scoped_fixture])


@st.composite
def layers(draw):
    B = draw(st.integers(1, 3))
    Hkv = draw(st.integers(1, 3))
    G = draw(st.sampled_from([1, 2, 4]))
    lens = draw(st.lists(st.integers(1, 300), min_size=B, max_size=B))
    bs = draw(st.lists(st.sampled_from([16, 32, 64]), min_size=Hkv, max_size=Hkv))
    budget = draw(st.integers(1, 400))
    const_channel = draw(st.booleans())
    ties = draw(st.booleans())
    seed = draw(st.integers(0, 2**16))
    w = W.PRESETS[0].scaled(batch=B, num_q_heads=Hkv * G, num_kv_heads=Hkv, head_dim=64, context=max(lens),
                            dtype="f32", token_budget=budget, needles_per_head=2, fixed_block_sizes=tuple(bs))
    x = W.make_layer(w, seq_lens=lens)
    rng = np.random.default_rng(seed)
    if const_channel:
        x.k_cache[:, :, :, int(rng.integers(0, 64))] = np.float32(0.75)
    if ties:
        # coarse keys: many blocks with identical centroids and scores
        x.k_cache[:] = np.round(x.k_cache[:] * 0.25).astype(np.float32)
    return x, budget


@SETTINGS
@given(layers())
def test_pipeline_properties(oracle_mod, case):
    x, budget = case
    c = oracle_mod.centroids(x.k_cache, x.page_table, x.seq_lens, x.block_size, "f32")
    qz = oracle_mod.quantize(c, x.seq_lens, x.block_size)
    s = oracle_mod.scores(x.q, qz, x.seq_lens, x.block_size, "f32")
    cap = oracle_mod.sel_capacity(x.seq_lens, x.block_size, budget)
    sel, cnt = oracle_mod.select(s, x.seq_lens, x.block_size, budget, cap)
    for b, h, r0, n in oracle_mod.block_rows(x.seq_lens, x.block_size):
        L, bs = int(x.seq_lens[b]), int(x.block_size[h])
        keys = W.contiguous_kv(x, "k", b)[h].astype(np.float64)
        # centroid: exact mean of the valid tokens of the last (possibly partial) block
        blk = keys[(n - 1) * bs:L]
        want = np.float32([math.fsum(blk[:, d]) / len(blk) for d in range(blk.shape[1])])
        np.testing.assert_array_equal(c[r0 + n - 1], want)
        # INT4: codes in range, error within scale / 2
        sc = qz.scale[b, h].astype(np.float64)
        chat = qz.codes[r0:r0 + n] * sc + qz.lo[b, h]
        assert qz.codes[r0:r0 + n].max() <= 15
        assert (np.abs(chat - c[r0:r0 + n]) <= sc / 2 * (1 + 1e-5) + 1e-6).all()
        # top-K: the budget rule, ascending unique indices, every kept score
        # >= every dropped one, ties at the threshold to the lower indices
        k = int(cnt[b, h])
        assert k == min(n, max(1, budget // bs))
        kept = sel[b, h, :k]
        assert (np.diff(kept) > 0).all() and kept.min() >= 0 and kept.max() < n
        sh = s[r0:r0 + n]
        dropped = np.setdiff1d(np.arange(n), kept)
        if len(dropped):
            tau = sh[kept].min()
            assert sh[dropped].max() <= tau
            tied_out = dropped[sh[dropped] == tau]
            tied_in = kept[sh[kept] == tau]
            if len(tied_out) and len(tied_in):
                assert tied_in.max() < tied_out.min()


@SETTINGS
@given(layers())
def test_all_blocks_is_dense_softmax(oracle_mod, case):
    """With a budget covering every block, attention is dense softmax over all
    L_b tokens (plain numpy, fp64)."""
    x, _ = case
    big = 1 << 20
    c = oracle_mod.centroids(x.k_cache, x.page_table, x.seq_lens, x.block_size, "f32")
    qz = oracle_mod.quantize(c, x.seq_lens, x.block_size)
    s = oracle_mod.scores(x.q, qz, x.seq_lens, x.block_size, "f32")
    cap = oracle_mod.sel_capacity(x.seq_lens, x.block_size, big)
    sel, cnt = oracle_mod.select(s, x.seq_lens, x.block_size, big, cap)
    sm = 0.125
    out, lse = oracle_mod.attend(x.q, x.k_cache, x.v_cache, x.page_table, x.seq_lens, x.block_size, sel, cnt, sm,
                                 "f32")
    B, Hq, D = x.q.shape
    G = Hq // x.k_cache.shape[1]
    for b in range(B):
        K = W.contiguous_kv(x, "k", b).astype(np.float64)
        V = W.contiguous_kv(x, "v", b).astype(np.float64)
        for i in range(Hq):
            z = sm * (K[i // G] @ x.q[b, i].astype(np.float64))
            m = z.max()
            p = np.exp(z - m)
            np.testing.assert_allclose(out[b, i], p @ V[i // G] / p.sum(), rtol=1e-9, atol=1e-12)
            assert abs(lse[b, i] - (m + math.log(p.sum()))) < 1e-9
