"""Parity of the offline block-size calibration on the GPU (through the C
ABI) with the oracle: per block size, the per-head recall that
abs_head_recall derives from the decode's log-sum-exps equals the oracle's
kept attention share on the GPU's own selection (fp32 caches: 1e-4
relative; bf16: 2e-3, from the lse tolerances of the attention parity);
end to end, calibrate_block_sizes recovers the map the synthetic layer
plants (scattered needles -> 16, 2-token runs -> 32, longer runs -> 64), as
the oracle's calibration does."""
import numpy as np
import pytest
import torch

from block_sparse_attention_abs_amd import abs as A
from block_sparse_attention_abs_amd import workload as W

pytestmark = pytest.mark.gpu
RUNS = [1, 2, 4, 64]
BUDGET = 1536


def _layer(dtype):
    w = W.PRESETS[1].scaled(batch=2, context=8192, token_budget=BUDGET, needles_per_head=64,
                            num_q_heads=4 * len(RUNS), num_kv_heads=len(RUNS), dtype=dtype)
    return W.make_layer(w, needle_runs=RUNS)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_head_recall_matches_oracle_mass(oracle_mod, dtype):
    x = _layer(dtype)
    B, Hq, D = x.q.shape
    Hkv = x.k_cache.shape[1]
    G = Hq // Hkv
    sm = float(np.float32(1.0 / np.sqrt(D)))
    print(f"[gpu calibration] head recall {dtype} lens={x.seq_lens.tolist()} runs={RUNS}", flush=True)
    base = A.PagedKV.from_host(Hq, x.k_cache, x.v_cache, x.page_table, x.seq_lens, x.block_size, x.dtype)
    q = A.upload(x.q, "cuda", x.dtype)
    out = torch.empty((B, Hq, D), dtype=A.torch_dtype(x.dtype), device="cuda")
    lse_full = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    lse_sel = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    recall = torch.empty((3, Hkv), dtype=torch.float32, device="cuda")
    tol = 1e-4 if dtype == "f32" else 2e-3
    for k, bs in enumerate((16, 32, 64)):
        layer = base.with_block_sizes(np.full(Hkv, bs, dtype=np.int32))
        cents = A.build_centroids(layer, A.Centroids.empty(layer))
        everything = int(x.seq_lens.max())
        for bud, lse in ((everything, lse_full), (BUDGET, lse_sel)):
            cap = layer.select_capacity(bud)
            sel = torch.empty((B, Hkv, cap), dtype=torch.int32, device="cuda")
            cnt = torch.empty((B, Hkv), dtype=torch.int32, device="cuda")
            A.score_select(layer, cents, q, bud, sel, cnt)
            A.sparse_decode(layer, q, sel, cnt, bud, sm, out, lse)
        A.abs_head_recall(layer.kv, int(lse_sel.data_ptr()), int(lse_full.data_ptr()), int(recall[k].data_ptr()),
                          A.current_stream())
        torch.cuda.synchronize()
        sel_h, cnt_h = sel.cpu().numpy(), cnt.cpu().numpy()
        mass = oracle_mod.attention_mass(x.q, x.k_cache, x.page_table, x.seq_lens, layer.block_size_host, sel_h,
                                         cnt_h, sm, x.dtype)
        want = mass.reshape(B, Hkv, G).mean(axis=(0, 2))
        got = recall[k].cpu().numpy().astype(np.float64)
        np.testing.assert_allclose(got, want, rtol=tol, atol=0)
        assert ((got > 0) & (got <= 1 + tol)).all()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_calibration_recovers_the_planted_map(oracle_mod, dtype):
    x = _layer(dtype)
    Hq, D = x.q.shape[1], x.q.shape[2]
    sm = float(np.float32(1.0 / np.sqrt(D)))
    print(f"[gpu calibration] end to end {dtype}", flush=True)
    kv = A.PagedKV.from_host(Hq, x.k_cache, x.v_cache, x.page_table, x.seq_lens, x.block_size, x.dtype)
    q = A.upload(x.q, "cuda", x.dtype)
    got_map, got_r = A.calibrate_block_sizes(kv, q, BUDGET, sm, threshold=0.95)
    R = np.array([oracle_mod.head_recall(x, bs, BUDGET, sm) for bs in (16, 32, 64)])
    want_map = oracle_mod.assign_block_sizes(R, 0.95)
    print(f"[gpu calibration] recall gpu {np.round(got_r, 4).tolist()} oracle {np.round(R, 4).tolist()}",
          flush=True)
    np.testing.assert_array_equal(want_map, [16, 32, 64, 64])
    np.testing.assert_array_equal(got_map, want_map)
    np.testing.assert_allclose(got_r, R, rtol=0.02, atol=0)
