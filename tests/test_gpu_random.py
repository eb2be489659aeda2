"""Seeded random layers through the whole path on the GPU (C ABI), against
the oracle: random batch, heads, group size (1 to 8, slots padded), head_dim,
dtype, block-size map, ragged lengths (partial pages and blocks), budget and
centroid format.  Each case checks the codes bit for bit, the selection under
the tie-band rule and the attention on the GPU's selection (rules of
gpu_pipeline.py), and abs_select_decode against the separate calls bit for
bit (the fused launch where the layer takes it)."""
import numpy as np
import pytest
import torch

from block_sparse_attention_abs_amd import abs as A
from block_sparse_attention_abs_amd import workload as W
from gpu_pipeline import check_attention, check_selection, codes_of_format, default_scale

pytestmark = pytest.mark.gpu
FORMATS = ["int4", "int4_sym", "int8", "int4_tensor", "bf16"]


def _case(seed):
    r = np.random.default_rng(1000 + seed)
    Hkv = int(r.choice([1, 2, 3, 4, 8]))
    G = int(r.choice([1, 2, 3, 4, 5, 6, 7, 8]))
    D = int(r.choice([64, 128]))
    dtype = str(r.choice(["f32", "bf16"]))
    B = int(r.integers(1, 6))
    lens = r.integers(1, 5000, B).tolist()
    bs = tuple(int(b) for b in r.choice([16, 32, 64], Hkv))
    budget = int(r.choice([1, 15, 64, 100, 512, 2048, 8192]))
    fmt = FORMATS[seed % len(FORMATS)]
    w = W.PRESETS[1].scaled(batch=B, num_q_heads=Hkv * G, num_kv_heads=Hkv, head_dim=D, dtype=dtype,
                            context=max(lens), token_budget=budget, needles_per_head=int(r.integers(0, 9)),
                            fixed_block_sizes=bs)
    return W.make_layer(w, seq_lens=lens, extra_pages=int(r.integers(0, 4))), budget, fmt


def _long_case(seed):
    """Long contexts (1K to 300K tokens): heads of up to 18,750 blocks, so the
    top-K launch's 1024-thread form and the fused launch's 32-key form run."""
    r = np.random.default_rng(9000 + seed)
    Hkv = int(r.choice([1, 2, 3, 4, 8]))
    G = int(r.choice([1, 2, 3, 4, 5, 6, 7, 8]))
    D = int(r.choice([64, 128]))
    dtype = str(r.choice(["f32", "bf16", "bf16"]))
    B = int(r.integers(1, 4))
    lens = r.integers(1000, 300000, B).tolist()
    bs = tuple(int(b) for b in r.choice([16, 32, 64], Hkv))
    budget = int(r.choice([64, 1024, 4096, 8192]))
    fmt = FORMATS[seed % len(FORMATS)]
    w = W.PRESETS[1].scaled(batch=B, num_q_heads=Hkv * G, num_kv_heads=Hkv, head_dim=D, dtype=dtype,
                            context=max(lens), token_budget=budget, needles_per_head=int(r.integers(0, 17)),
                            fixed_block_sizes=bs)
    return W.make_layer(w, seq_lens=lens, extra_pages=int(r.integers(0, 4))), budget, fmt


@pytest.mark.parametrize("seed", range(40))
def test_random_layer(oracle_mod, seed):
    _check_case(oracle_mod, seed, *_case(seed))


@pytest.mark.parametrize("seed", range(6))
def test_random_long_layer(oracle_mod, seed):
    _check_case(oracle_mod, seed, *_long_case(seed))


def _check_case(oracle_mod, seed, x, budget, fmt):
    B, Hq, D = x.q.shape
    Hkv = x.k_cache.shape[1]
    print(f"[gpu random] seed={seed} B={B} Hq={Hq} Hkv={Hkv} D={D} {x.dtype} lens={x.seq_lens.tolist()} "
          f"bs={x.block_size.tolist()} budget={budget} fmt={fmt}", flush=True)
    kv = A.PagedKV.from_host(Hq, x.k_cache, x.v_cache, x.page_table, x.seq_lens, x.block_size, x.dtype)
    cents = A.build_centroids(kv, A.Centroids.empty(kv, fmt))
    q = A.upload(x.q, "cuda", x.dtype)
    cap = kv.select_capacity(budget)
    sel = torch.full((B, Hkv, cap), -1, dtype=torch.int32, device="cuda")
    cnt = torch.zeros((B, Hkv), dtype=torch.int32, device="cuda")
    A.score_select(kv, cents, q, budget, sel, cnt)
    sm = default_scale(D)
    out = torch.empty((B, Hq, D), dtype=A.torch_dtype(x.dtype), device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    A.sparse_decode(kv, q, sel, cnt, budget, sm, out, lse)
    fsel = torch.full((B, Hkv, cap), -1, dtype=torch.int32, device="cuda")
    fcnt = torch.zeros((B, Hkv), dtype=torch.int32, device="cuda")
    fout = torch.empty((B, Hq, D), dtype=A.torch_dtype(x.dtype), device="cuda")
    flse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    A.select_decode(kv, cents, q, budget, sm, fsel, fcnt, fout, flse)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(fcnt.cpu().numpy(), cnt.cpu().numpy())
    fs, ss = fsel.cpu().numpy(), sel.cpu().numpy()
    for (b, h), k in np.ndenumerate(cnt.cpu().numpy()):
        np.testing.assert_array_equal(fs[b, h, :k], ss[b, h, :k])
    np.testing.assert_array_equal(fout.float().cpu().numpy(), out.float().cpu().numpy())
    np.testing.assert_array_equal(flse.cpu().numpy(), lse.cpu().numpy())

    c = oracle_mod.centroids(x.k_cache, x.page_table, x.seq_lens, x.block_size, x.dtype)
    qf = oracle_mod.quantize_fmt(c, x.seq_lens, x.block_size, fmt)
    np.testing.assert_array_equal(codes_of_format(cents.codes.cpu().numpy(), fmt), qf.codes)
    np.testing.assert_array_equal(cents.scale.cpu().numpy(), qf.scale)
    np.testing.assert_array_equal(cents.lo.cpu().numpy(), qf.lo)
    s = oracle_mod.scores_dense(x.q, qf.deq, x.seq_lens, x.block_size, x.dtype)
    sel_h, cnt_h = sel.cpu().numpy(), cnt.cpu().numpy()
    check_selection(oracle_mod, x, qf, s, sel_h, cnt_h, budget)
    ref_out, ref_lse = oracle_mod.attend(x.q, x.k_cache, x.v_cache, x.page_table, x.seq_lens, x.block_size, sel_h,
                                         cnt_h, sm, x.dtype)
    check_attention(out.float().cpu().numpy(), lse.cpu().numpy(), ref_out, ref_lse, x.dtype)
