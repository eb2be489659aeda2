"""abs_select_decode (scores, then the top-K inside the split decode launch)
against the two separate calls and against the oracle, through the C ABI.

The fused launch runs the same selection (the top-K launch's code, 512
threads per head) and the same decode arithmetic on the same pages, so sel,
sel_count, out and lse must equal the separate calls' bit for bit.
Layers the fused launch does not serve (fp32, head_dim 64, 8-head groups,
16384 blocks in every head, and small layers whose split decode holds
fewer than 8 pages per workgroup) run the separate launches and must give
the same results too; each case asserts which form it gets.  Against the oracle: the selection rule and the attention
tolerances of gpu_pipeline.
"""
import numpy as np
import pytest
import torch

from block_sparse_attention_abs_amd import abs as A
from block_sparse_attention_abs_amd import workload as W
from gpu_pipeline import GpuLayer, check_attention, check_selection, default_scale, to_host_f32

pytestmark = pytest.mark.gpu

P = W.PRESETS


def _case(name):
    if name == "b2-16k":                       # 1024 blocks at most: 4 keys per thread
        return W.make_layer(P[2].scaled(batch=2, context=16384))
    if name == "ragged-4k":
        return W.make_layer(P[1].scaled(batch=3, context=4096, token_budget=512), seq_lens=[4096, 3001, 77])
    if name == "b1-128k":                      # 8192 blocks in the block-size-16 head: 16 keys per thread
        return W.make_layer(P[3].scaled(batch=1))
    if name == "b1-256k":                      # 16384 blocks in that head: 32 keys per thread
        return W.make_layer(P[3].scaled(batch=1, context=262144))
    if name == "b1-64k-bs16":                  # 4096 blocks in every head: 8 keys per thread
        return W.make_layer(P[1].scaled(context=65536, fixed_block_sizes=(16,) * 8))
    if name == "gqa2":
        return W.make_layer(P[1].scaled(num_q_heads=16, batch=2, context=6000), seq_lens=[6000, 2500])
    if name == "gqa1":                         # one query head per KV head
        return W.make_layer(P[1].scaled(num_q_heads=8, batch=2, context=5000), seq_lens=[5000, 1800])
    if name == "b1-128k-mixed":                # 512 threads; heads of 8192, 4096 and 2048 blocks: 16, 8 and 4 keys
        return W.make_layer(P[3].scaled(batch=1, fixed_block_sizes=(16, 32, 64, 32, 64, 16, 32, 64)))
    if name == "dense-short":                  # fused; the short sequence has K = N (every block selected)
        return W.make_layer(P[2].scaled(batch=2, context=16384), seq_lens=[16384, 500])
    if name == "budget-covers":                # K = N: every block selected (a small layer: separate launches)
        return W.make_layer(P[1].scaled(batch=2, context=1000, token_budget=4096), seq_lens=[1000, 333])
    # not served by the fused launch
    if name == "f32":
        return W.make_layer(P[1].scaled(dtype="f32", batch=2, context=3000))
    if name == "d64":
        return W.make_layer(P[1].scaled(head_dim=64, batch=2, context=3000))
    if name == "gqa8":
        return W.make_layer(P[1].scaled(num_q_heads=16, num_kv_heads=2, batch=2, context=3000))
    if name == "b1-256k-bs16":                 # 16384 blocks in every head
        return W.make_layer(P[1].scaled(context=262144, fixed_block_sizes=(16,) * 8, token_budget=4096))
    raise KeyError(name)


CASES = ["b2-16k", "ragged-4k", "b1-128k", "b1-256k", "b1-64k-bs16", "gqa2", "gqa1", "b1-128k-mixed",
         "dense-short", "budget-covers", "f32", "d64", "gqa8", "b1-256k-bs16"]
# layers abs_select_decode runs as the separate launches (on a device of 256 compute units)
SEPARATE = {"ragged-4k", "budget-covers", "f32", "d64", "gqa8", "b1-256k-bs16"}


def _fused(g, budget, sm, ws):
    x = g.x
    B, Hq, D = x.q.shape
    cap = g.kv.select_capacity(budget)
    sel = torch.full((B, x.k_cache.shape[1], cap), -1, dtype=torch.int32, device="cuda")
    cnt = torch.zeros((B, x.k_cache.shape[1]), dtype=torch.int32, device="cuda")
    out = torch.empty((B, Hq, D), dtype=A.torch_dtype(x.dtype), device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    A.select_decode(g.kv, g.cents, g.q, budget, sm, sel, cnt, out, lse, ws=ws)
    torch.cuda.synchronize()
    return sel.cpu().numpy(), cnt.cpu().numpy(), to_host_f32(out), lse.cpu().numpy()


def _same(a, b):
    sel_a, cnt_a, out_a, lse_a = a
    sel_b, cnt_b, out_b, lse_b = b
    np.testing.assert_array_equal(cnt_a, cnt_b)
    for (bb, h), k in np.ndenumerate(cnt_a):
        np.testing.assert_array_equal(sel_a[bb, h, :k], sel_b[bb, h, :k])
    np.testing.assert_array_equal(out_a, out_b)
    np.testing.assert_array_equal(lse_a, lse_b)


@pytest.mark.parametrize("case", CASES)
def test_fused_equals_separate_calls_and_oracle(oracle_mod, case):
    x = _case(case)
    budget = x.workload.token_budget
    sm = default_scale(x.q.shape[2])
    print(f"[gpu select_decode] {case}: B={x.q.shape[0]} Hq={x.q.shape[1]} Hkv={x.k_cache.shape[1]} "
          f"D={x.q.shape[2]} lens={x.seq_lens.tolist()} bs={x.block_size.tolist()} {x.dtype}", flush=True)
    g = GpuLayer(x)
    plan = g.kv.launch_plan(budget)
    if plan["compute_units"] == 256:               # the launch choice depends on the device's CU count
        assert plan["fused"] == (0 if case in SEPARATE else 1), plan
    g.build()
    sel, cnt = g.select(budget)
    out, lse = g.decode(sel, cnt, budget, sm)
    torch.cuda.synchronize()
    sep = (sel.cpu().numpy(), cnt.cpu().numpy(), to_host_f32(out), lse.cpu().numpy())
    ws = A.workspace(g.kv.workspace_bytes(budget, A.ABS_OP_SELECT_DECODE))
    first = _fused(g, budget, sm, ws)
    _same(first, sep)
    _same(_fused(g, budget, sm, ws), first)        # the same workspace again: arrival counters back at zero
    # against the oracle, from the raw inputs
    ref = oracle_mod.run(x, sm_scale=sm, budget=budget)
    check_selection(oracle_mod, x, ref.quant, ref.scores, first[0], first[1], budget)
    o, l = oracle_mod.attend(x.q, x.k_cache, x.v_cache, x.page_table, x.seq_lens, x.block_size, first[0],
                             first[1], sm, x.dtype)
    check_attention(first[2], first[3], o, l, x.dtype)
    del g, ws
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name,context,K,n10,n5", [("few-below", 16384, 128, 100, 50),
                                                    ("edge-64", 16384, 128, 100, 64),
                                                    ("edge-65", 16384, 128, 100, 65),
                                                    ("crowded", 16384, 128, 100, 200),
                                                    ("overflow", 16384, 128, 0, 600),
                                                    ("wide-crowded", 65536, 128, 100, 200),
                                                    ("wide-overflow", 65536, 128, 0, 600)])
def test_fused_ties(name, context, K, n10, n5):
    """Runs of equal scores at the threshold (the construction of
    test_gpu_topk_ties, with K = 128 so that each head's 128 pages give the
    split decode 8 per workgroup and the layer takes the fused launch): the
    in-decode top-K takes the same ranked path (at most 64 tied
    candidates), LDS ranking (65-512) or radix path (more) as the top-K
    launch."""
    from test_gpu_topk_ties import _layer
    x, groups = _layer(context, K, n10, n5, "bf16", seed=context + n5)
    budget = 16 * K
    sm = default_scale(x.q.shape[2])
    print(f"[gpu select_decode] ties {name}", flush=True)
    g = GpuLayer(x)
    plan = g.kv.launch_plan(budget)
    if plan["compute_units"] == 256:
        assert plan["fused"] == 1, plan
    g.build()
    sel, cnt = g.select(budget)
    out, lse = g.decode(sel, cnt, budget, sm)
    torch.cuda.synchronize()
    sep = (sel.cpu().numpy(), cnt.cpu().numpy(), to_host_f32(out), lse.cpu().numpy())
    ws = A.workspace(g.kv.workspace_bytes(budget, A.ABS_OP_SELECT_DECODE))
    fused = _fused(g, budget, sm, ws)
    _same(fused, sep)
    for (b, h), (s10, s5) in groups.items():
        want = np.sort(np.concatenate([s10, s5[:K - len(s10)]]))
        np.testing.assert_array_equal(fused[0][b, h, :K], want)


@pytest.mark.parametrize("case", ["gqa2", "ragged-4k"])
def test_fused_in_a_graph_replays_like_eager(case):
    """abs_select_decode captured in a HIP graph (the fused launch for gqa2,
    the separate launches for the small ragged layer) and replayed: every
    replay equals the eager call."""
    x = _case(case)
    budget = x.workload.token_budget
    sm = default_scale(x.q.shape[2])
    g = GpuLayer(x)
    plan = g.kv.launch_plan(budget)
    if plan["compute_units"] == 256:
        assert plan["fused"] == (0 if case in SEPARATE else 1), plan
    g.build()
    B, Hq, D = x.q.shape
    cap = g.kv.select_capacity(budget)
    sel = torch.zeros((B, x.k_cache.shape[1], cap), dtype=torch.int32, device="cuda")
    cnt = torch.zeros((B, x.k_cache.shape[1]), dtype=torch.int32, device="cuda")
    out = torch.empty((B, Hq, D), dtype=A.torch_dtype(x.dtype), device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    ws = A.workspace(g.kv.workspace_bytes(budget, A.ABS_OP_SELECT_DECODE))
    A.select_decode(g.kv, g.cents, g.q, budget, sm, sel, cnt, out, lse, ws=ws)
    torch.cuda.synchronize()
    eager = (sel.clone(), cnt.clone(), out.clone(), lse.clone())
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            A.select_decode(g.kv, g.cents, g.q, budget, sm, sel, cnt, out, lse, ws=ws,
                            stream=int(s.cuda_stream))
    torch.cuda.synchronize()
    for _ in range(3):
        out.zero_()
        lse.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager[2]) and torch.equal(lse, eager[3]) and torch.equal(cnt, eager[1])
        for (b, h), k in np.ndenumerate(eager[1].cpu().numpy()):
            assert torch.equal(sel[b, h, :k], eager[0][b, h, :k])


@pytest.mark.parametrize("case", ["b2-16k", "b1-128k", "ragged-4k", "f32"])
def test_estimate_then_topk_decode_equals_select_decode(case):
    """abs_estimate + abs_topk_decode (the two halves of the per-stage split)
    on one workspace make the launches of abs_select_decode: sel, sel_count,
    out and lse bit for bit, on a fused layer and on layers that take the
    separate launches; a workspace filled with stale bytes needs no reset."""
    x = _case(case)
    budget = x.workload.token_budget
    sm = default_scale(x.q.shape[2])
    g = GpuLayer(x)
    g.build()
    ws = A.workspace(g.kv.workspace_bytes(budget, A.ABS_OP_SELECT_DECODE))
    want = _fused(g, budget, sm, ws)
    B, Hq, D = x.q.shape
    cap = g.kv.select_capacity(budget)
    stale = torch.full((ws.numel(),), 0x7F, dtype=torch.uint8, device="cuda")
    sel = torch.full((B, x.k_cache.shape[1], cap), -1, dtype=torch.int32, device="cuda")
    cnt = torch.zeros((B, x.k_cache.shape[1]), dtype=torch.int32, device="cuda")
    out = torch.empty((B, Hq, D), dtype=A.torch_dtype(x.dtype), device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    st = A.current_stream()
    A.abs_estimate(g.kv.kv, g.kv.bmap, g.cents.desc, g.q.data_ptr(), budget, stale.data_ptr(), stale.numel(), st)
    A.abs_topk_decode(g.kv.kv, g.kv.bmap, g.q.data_ptr(), budget, sm, sel.data_ptr(), cap, cnt.data_ptr(),
                      out.data_ptr(), lse.data_ptr(), stale.data_ptr(), stale.numel(), st)
    torch.cuda.synchronize()
    _same((sel.cpu().numpy(), cnt.cpu().numpy(), to_host_f32(out), lse.cpu().numpy()), want)
