"""Parity of the HIP path (through the C ABI) with the CPU oracle on the GPU.

Stage-isolated checks feed each stage's oracle the GPU's own upstream
results (GPU codes into the oracle's scoring, GPU selection into the
oracle's attention), so each kernel is judged on the same inputs; the
end-to-end check runs the oracle from the raw inputs.  Rules and tolerances
are in gpu_pipeline.py.
"""
import dataclasses

import numpy as np
import pytest
import torch

from block_sparse_attention_abs_amd import workload as W
from gpu_pipeline import (GpuLayer, attention_vs_own_selection, check_attention, check_selection, default_scale,
                          oracle_quant_from_gpu)

pytestmark = pytest.mark.gpu

P = W.PRESETS


def _case(name):
    if name == "tiny":
        return W.make_layer(P[0])
    if name == "tiny-ragged":
        return W.make_layer(P[0].scaled(batch=3), seq_lens=[2048, 1001, 17])
    if name == "llama-4k-ragged":
        return W.make_layer(P[1].scaled(batch=2, context=4096, token_budget=512), seq_lens=[4096, 3001])
    if name == "llama-16k-b2":
        return W.make_layer(P[2].scaled(batch=2, context=16384))
    if name == "mha-d128-f32":
        return W.make_layer(P[1].scaled(num_q_heads=8, num_kv_heads=8, dtype="f32", context=1500, token_budget=256))
    if name == "gqa8-d64-bf16":
        return W.make_layer(P[1].scaled(num_q_heads=16, num_kv_heads=2, head_dim=64, context=3000,
                                        token_budget=512, batch=2), seq_lens=[3000, 2222])
    raise KeyError(name)


CASES = ["tiny", "tiny-ragged", "llama-4k-ragged", "llama-16k-b2", "mha-d128-f32", "gqa8-d64-bf16"]


@pytest.fixture(scope="module")
def runs(oracle_mod):
    cache = {}

    def get(name):
        if name not in cache:
            x = _case(name)
            print(f"[gpu parity] case {name}: B={x.q.shape[0]} Hq={x.q.shape[1]} Hkv={x.k_cache.shape[1]} "
                  f"D={x.q.shape[2]} lens={x.seq_lens.tolist()} bs={x.block_size.tolist()} {x.dtype}", flush=True)
            g = GpuLayer(x)
            sm = default_scale(x.q.shape[2])
            res = g.run(x.workload.token_budget, sm)
            cache[name] = (x, g, res, sm)
        return cache[name]

    return get


@pytest.mark.parametrize("case", CASES)
def test_build_is_bit_exact(runs, oracle_mod, case):
    x, _, r, _ = runs(case)
    c = oracle_mod.centroids(x.k_cache, x.page_table, x.seq_lens, x.block_size, x.dtype)
    qz = oracle_mod.quantize(c, x.seq_lens, x.block_size)
    np.testing.assert_array_equal(r.scale, qz.scale)
    np.testing.assert_array_equal(r.lo, qz.lo)
    np.testing.assert_array_equal(r.codes, qz.codes)


@pytest.mark.parametrize("case", CASES)
def test_select_stage(runs, oracle_mod, case):
    x, _, r, _ = runs(case)
    qz = oracle_quant_from_gpu(oracle_mod, r)
    s = oracle_mod.scores(x.q, qz, x.seq_lens, x.block_size, x.dtype)
    check_selection(oracle_mod, x, qz, s, r.sel, r.count, x.workload.token_budget)


@pytest.mark.parametrize("case", CASES)
def test_decode_stage(runs, oracle_mod, case):
    x, _, r, sm = runs(case)
    out, lse = oracle_mod.attend(x.q, x.k_cache, x.v_cache, x.page_table, x.seq_lens, x.block_size, r.sel, r.count,
                                 sm, x.dtype)
    check_attention(r.out, r.lse, out, lse, x.dtype)


@pytest.mark.parametrize("case", CASES)
def test_end_to_end(runs, oracle_mod, case):
    """The oracle from the raw inputs: selections under the tie-band rule,
    outputs against the oracle run over the GPU's selection (so a legitimate
    near-tie swap is not scored as an attention error); the difference
    against the oracle's own selection is reported, and held to the same
    tolerances when the two selections agree."""
    x, _, r, sm = runs(case)
    ref = oracle_mod.run(x, sm_scale=sm)
    swaps = check_selection(oracle_mod, x, ref.quant, ref.scores, r.sel, r.count, x.workload.token_budget)
    out, lse = oracle_mod.attend(x.q, x.k_cache, x.v_cache, x.page_table, x.seq_lens, x.block_size, r.sel, r.count,
                                 sm, x.dtype)
    check_attention(r.out, r.lse, out, lse, x.dtype)
    own = attention_vs_own_selection(r.out, ref)
    print(f"[gpu parity] {case}: {swaps} tie-band swaps; against the oracle's own selection {own}", flush=True)
    if swaps == 0:
        check_attention(r.out, r.lse, ref.out, ref.lse, x.dtype)


def _run_and_compare(oracle_mod, x, budget, sm=None):
    sm = default_scale(x.q.shape[2]) if sm is None else sm
    r = GpuLayer(x).run(budget, sm)
    ref = oracle_mod.run(x, sm_scale=sm, budget=budget)
    np.testing.assert_array_equal(r.codes, ref.quant.codes)
    check_selection(oracle_mod, x, ref.quant, ref.scores, r.sel, r.count, budget)
    out, lse = oracle_mod.attend(x.q, x.k_cache, x.v_cache, x.page_table, x.seq_lens, x.block_size, r.sel, r.count,
                                 sm, x.dtype)
    check_attention(r.out, r.lse, out, lse, x.dtype)
    return r, ref


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_budget_covering_context_is_dense_attention(oracle_mod, dtype):
    x = W.make_layer(P[1].scaled(batch=2, context=1000, dtype=dtype), seq_lens=[1000, 333])
    r, ref = _run_and_compare(oracle_mod, x, budget=1 << 20)
    n = [[(int(L) + int(bs) - 1) // int(bs) for bs in x.block_size] for L in x.seq_lens]
    assert r.count.tolist() == n
    check_attention(r.out, r.lse, ref.out, ref.lse, dtype)


@pytest.mark.parametrize("bs", [(16,) * 8, (16, 64, 32, 64, 16, 32, 64, 64)])
def test_many_score_tiles_ragged(oracle_mod, bs):
    """More score tiles than the launch can list (the per-sequence grid):
    40 ragged sequences, some far shorter than the longest, so workgroups
    past their blocks must leave without writing."""
    rng = np.random.default_rng(11)
    lens = [32768, 1, 17, 4096, 255, 256, 257] + rng.integers(1, 32769, 33).tolist()
    x = W.make_layer(P[1].scaled(batch=len(lens), context=32768, token_budget=1024, needles_per_head=8,
                                 fixed_block_sizes=bs), seq_lens=lens)
    tiles = sum(-(-(-(-L // b)) // 256) for L in lens for b in bs)
    print(f"[gpu parity] many score tiles: {tiles} tiles, bs={bs}", flush=True)
    assert tiles > 512
    _run_and_compare(oracle_mod, x, budget=1024)


def test_tiny_lengths_partial_pages_and_blocks(oracle_mod):
    lens = [1, 15, 16, 17, 33, 63, 64, 65, 100]
    x = W.make_layer(P[1].scaled(batch=len(lens), context=100, needles_per_head=2), seq_lens=lens)
    _run_and_compare(oracle_mod, x, budget=64)


def test_budget_below_block_size_keeps_one_block(oracle_mod):
    x = W.make_layer(P[1].scaled(batch=2, context=2048, needles_per_head=4))
    r, _ = _run_and_compare(oracle_mod, x, budget=8)
    assert (r.count == 1).all()


def test_equal_scores_take_lowest_indices(oracle_mod):
    x = W.make_layer(P[1].scaled(batch=2, context=1000, dtype="f32"), seq_lens=[1000, 640], needles=False)
    x.k_cache[:] = np.float32(0.5)
    r, ref = _run_and_compare(oracle_mod, x, budget=128)
    assert (r.codes == 0).all() and (r.scale == 0).all()
    for (b, h), k in np.ndenumerate(r.count):
        assert r.sel[b, h, :k].tolist() == list(range(k))


def test_page_table_invariance_and_determinism():
    w = P[1].scaled(batch=3, context=3000, needles_per_head=4)
    a = W.make_layer(w, seq_lens=[3000, 1234, 77], shuffle_pages=True, extra_pages=5)
    b = W.make_layer(w, seq_lens=[3000, 1234, 77], shuffle_pages=False, extra_pages=5)
    sm = default_scale(128)
    ga = GpuLayer(a)
    ra = ga.run(2048, sm)
    ra2 = ga.run(2048, sm)
    rb = GpuLayer(b).run(2048, sm)
    for f in ("codes", "scale", "lo", "sel", "count", "out", "lse"):
        np.testing.assert_array_equal(getattr(ra, f), getattr(ra2, f))
        np.testing.assert_array_equal(getattr(ra, f), getattr(rb, f))


def test_largest_head_65536_blocks(oracle_mod):
    """The largest supported block count per head (1M tokens at block size 16)."""
    w = P[1].scaled(num_q_heads=4, num_kv_heads=1, context=(1 << 20), fixed_block_sizes=(16,), token_budget=4096)
    x = W.make_layer(w)
    _run_and_compare(oracle_mod, x, budget=4096)


# The launch shape abs_select_decode takes for each full-size workload on an
# MI355X (256 compute units): (splits, pages per workgroup, double-buffered).
FULL_SIZE_PLAN = {1: (16, 8, 0), 2: (2, 64, 1), 3: (8, 32, 1), 4: (4, 32, 1)}


@pytest.mark.parametrize("cfg,layer", [(1, 0), (2, 0), (3, 0), (4, 0), (4, 17), (4, 35)])
def test_full_size_sampled(oracle_mod, cfg, layer):
    """Full-size workload (one layer of it) in the benchmark's launch
    configuration: the separate calls, then abs_select_decode (the call the
    benchmark times, top-K inside the decode launch), which must give the
    same sel, sel_count, out and lse bit for bit; the oracle recomputes the
    first and last sequence on their own."""
    w = P[cfg]
    x = W.make_layer(w, layer)
    print(f"[gpu parity] full size cfg {cfg} layer {layer}: {w.name} bs={x.block_size.tolist()}", flush=True)
    _full_size_check(oracle_mod, w, x, f"cfg {cfg} layer {layer}", FULL_SIZE_PLAN[cfg])


def test_fused_past_4gib_of_cache(oracle_mod):
    """128K x 16 with 8192 spare pages in the pool: the K and V caches are
    4.25 GiB each, and the shuffled page table puts selected pages past the
    4 GiB mark (byte offsets above 2^32).  The layer takes the fused launch
    at two split workgroups per compute unit (4 splits of 64 pages, 512
    workgroups); checked as the full-size workloads are."""
    w = P[3].scaled(batch=16)
    x = W.make_layer(w, extra_pages=8192)
    print(f"[gpu parity] 128K x 16 over 4 GiB: pool {x.k_cache.shape[0]} pages, "
          f"{x.k_cache.nbytes / 2**30:.2f} GiB per cache", flush=True)
    sel, cnt = _full_size_check(oracle_mod, w, x, "128K x 16 over 4 GiB", (4, 64, 1))
    Hkv = w.num_kv_heads
    top = 0
    for (b, h), k in np.ndenumerate(cnt):
        bs = int(x.block_size[h])
        for j in sel[b, h, :k]:
            end = min((int(j) + 1) * bs, int(x.seq_lens[b]))           # the block's tokens: j bs .. end - 1
            for pg in range(int(j) * bs // 16, (end + 15) // 16):
                top = max(top, (int(x.page_table[b, pg]) * Hkv + h + 1) * 16 * w.head_dim * 2)
    assert top > 2**32, top


def _full_size_check(oracle_mod, w, x, label, want_plan):
    from block_sparse_attention_abs_amd import abs as A
    sm = default_scale(w.head_dim)
    g = GpuLayer(x)
    plan = g.kv.launch_plan(w.token_budget)
    if plan["compute_units"] == 256:
        assert (plan["splits"], plan["pages_per_wg"], plan["pipelined"]) == want_plan, plan
        assert plan["fused"] == 1, plan
    r = g.run(w.token_budget, sm)
    B, Hq, D = x.q.shape
    cap = g.kv.select_capacity(w.token_budget)
    sel = torch.full((B, w.num_kv_heads, cap), -1, dtype=torch.int32, device="cuda")
    cnt = torch.zeros((B, w.num_kv_heads), dtype=torch.int32, device="cuda")
    out = torch.empty((B, Hq, D), dtype=A.torch_dtype(x.dtype), device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    A.select_decode(g.kv, g.cents, g.q, w.token_budget, sm, sel, cnt, out, lse)
    torch.cuda.synchronize()
    fsel, fcnt = sel.cpu().numpy(), cnt.cpu().numpy()
    np.testing.assert_array_equal(fcnt, r.count)
    for (b, h), k in np.ndenumerate(r.count):
        np.testing.assert_array_equal(fsel[b, h, :k], r.sel[b, h, :k])
    np.testing.assert_array_equal(out.float().cpu().numpy(), r.out)
    np.testing.assert_array_equal(lse.cpu().numpy(), r.lse)
    off = g.kv.centroid_off.cpu().numpy()
    for b in sorted({0, w.batch - 1}):
        xb = dataclasses.replace(x, q=x.q[b:b + 1], page_table=x.page_table[b:b + 1], seq_lens=x.seq_lens[b:b + 1])
        ref = oracle_mod.run(xb, sm_scale=sm)
        r0, r1 = off[b * w.num_kv_heads], off[(b + 1) * w.num_kv_heads]
        np.testing.assert_array_equal(r.codes[r0:r1], ref.quant.codes)
        np.testing.assert_array_equal(r.scale[b], ref.quant.scale[0])
        np.testing.assert_array_equal(r.lo[b], ref.quant.lo[0])
        check_selection(oracle_mod, xb, ref.quant, ref.scores, r.sel[b:b + 1], r.count[b:b + 1], w.token_budget)
        o, l = oracle_mod.attend(xb.q, x.k_cache, x.v_cache, xb.page_table, xb.seq_lens, x.block_size,
                                 r.sel[b:b + 1], r.count[b:b + 1], sm, x.dtype)
        mx, mean = check_attention(r.out[b:b + 1], r.lse[b:b + 1], o, l, x.dtype)
        own = attention_vs_own_selection(r.out[b:b + 1], ref)
        print(f"[gpu parity] {label} seq {b}: max/mean |out - oracle| {mx:.2e}/{mean:.2e}; "
              f"against the oracle's own selection {own}", flush=True)
    del g
    torch.cuda.empty_cache()
    return r.sel, r.count


def test_decode_repeats_bit_identical():
    """Split partials are handed to the merge launch through the workspace;
    the merge order is fixed, so 200 back-to-back calls on one workspace
    must agree bit for bit."""
    from block_sparse_attention_abs_amd import abs as A
    w = P[2].scaled(batch=4, context=16384)
    x = W.make_layer(w)
    g = GpuLayer(x)
    g.build()
    sel, cnt = g.select(w.token_budget)
    sm = default_scale(w.head_dim)
    B, Hq, D = x.q.shape
    ws = A.workspace(g.kv.workspace_bytes(w.token_budget, A.ABS_OP_DECODE))
    outs = []
    for _ in range(200):
        out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device="cuda")
        A.sparse_decode(g.kv, g.q, sel, cnt, w.token_budget, sm, out, ws=ws)
        outs.append(out)
    torch.cuda.synchronize()
    ref = outs[0].view(torch.int16)
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int16), ref)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_split_count_invariance(oracle_mod, dtype):
    """One sequence alone (many small splits) and the same sequence repeated 8
    times in a batch whose rows share its pages (few large, double-buffered
    splits): every copy's output equals the single run within fp32 merge
    rounding (bf16: one output ulp), and all 8 copies agree bit for bit."""
    w = P[1].scaled(context=8192, token_budget=1024, dtype=dtype)
    x = W.make_layer(w)
    sm = default_scale(128)
    r1 = GpuLayer(x).run(w.token_budget, sm)
    rep = 8
    xb = dataclasses.replace(x, q=np.repeat(x.q, rep, axis=0), page_table=np.repeat(x.page_table, rep, axis=0),
                             seq_lens=np.repeat(x.seq_lens, rep))
    r8 = GpuLayer(xb).run(w.token_budget, sm)
    assert (r8.count == r1.count).all()
    for b in range(rep):
        np.testing.assert_array_equal(r8.sel[b], r1.sel[0])
        np.testing.assert_array_equal(r8.out[b], r8.out[0])
    d = np.abs(r8.out[0].astype(np.float64) - r1.out[0])
    if dtype == "f32":
        assert d.max() <= 2e-6, d.max()
    else:
        assert (d <= np.abs(r1.out[0]) * 2.0 ** -7 + 1e-6).all(), d.max()
    assert np.abs(r8.lse[0] - r1.lse[0]).max() <= 1e-5
