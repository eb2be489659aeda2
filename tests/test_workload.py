"""The seeded input generator: shapes, determinism, and the structure the
workloads promise (outlier key channels, planted needles at cos 0.9 with the
group query, a shuffled page table, the block-size mix)."""
import numpy as np

from block_sparse_attention_abs_amd import workload as W


def test_deterministic_and_paged():
    w = W.PRESETS[0]
    a, b = W.make_layer(w), W.make_layer(w)
    for f in ("q", "k_cache", "v_cache", "page_table", "block_size", "needle_pos"):
        np.testing.assert_array_equal(getattr(a, f), getattr(b, f))
    assert a.k_cache.shape == (2048 // 16, 2, 16, 64) and a.k_cache.dtype == np.float32
    pt = a.page_table[0]
    assert sorted(pt.tolist()) == list(range(128)) and pt.tolist() != list(range(128))


def test_needles_and_outliers():
    w = W.PRESETS[0]
    x = W.make_layer(w)
    qf = W.to_f32(x.q, w.dtype).astype(np.float64)
    keys = W.contiguous_kv(x, "k", 0).astype(np.float64)
    for h in range(w.num_kv_heads):
        qbar = qf[0, h * w.group:(h + 1) * w.group].sum(0)
        for p in x.needle_pos[0, h]:
            k = keys[h, p]
            cos = k @ qbar / np.linalg.norm(k) / np.linalg.norm(qbar)
            assert abs(cos - W.NEEDLE_COS) < 1e-5
        rms = np.sqrt((keys[h] ** 2).mean(0))
        assert (rms > 5).sum() == W.OUTLIER_CHANNELS


def test_block_mix_and_ragged_padding():
    sizes = np.concatenate([W.block_sizes_for(W.PRESETS[4], l) for l in range(36)])
    frac = [(sizes == s).mean() for s in (16, 32, 64)]
    assert abs(frac[0] - .25) < .08 and abs(frac[1] - .25) < .08 and abs(frac[2] - .5) < .1
    w = W.PRESETS[1].scaled(batch=2, context=100, needles_per_head=2)
    x = W.make_layer(w, seq_lens=[100, 17])
    assert x.page_table.shape == (2, 7) and (x.page_table[1, 2:] == -1).all()
    last = x.k_cache[x.page_table[1, 1]]
    assert (W.bf16_bits_to_f32(last[:, 1:]) == W.PAD_SENTINEL).all()


def test_bf16_rounding_is_nearest_even():
    x = np.float32([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -3.140625, 65504.0])
    got = W.bf16_bits_to_f32(W.f32_to_bf16_bits(x))
    np.testing.assert_array_equal(got, np.float32([1.0, 1.0, 1.0 + 2 ** -6, -3.140625, 65536.0]))
