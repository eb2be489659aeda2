"""The decode step captured in a HIP graph (as bench.py times it): build,
select and decode recorded once, replayed several times with eager work
and synchronizations in between; every replay must give the eager result
bit for bit (the decode's arrival counters are reset by the merging
workgroup, so the graph needs no clearing node), and the eager result
matches the oracle."""
import numpy as np
import pytest
import torch

from block_sparse_attention_abs_amd import abs as A
from block_sparse_attention_abs_amd import workload as W
from gpu_pipeline import GpuLayer, check_attention, default_scale

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,cfg", [("bf16", 2), ("f32", 1)])
def test_graph_replays_match_eager(oracle_mod, dtype, cfg):
    w = W.PRESETS[cfg].scaled(batch=4, context=8192, dtype=dtype, token_budget=1024)
    x = W.make_layer(w)
    print(f"[gpu graph] {dtype} cfg{cfg} B={w.batch} ctx={w.context}", flush=True)
    g = GpuLayer(x)
    budget, sm = w.token_budget, default_scale(w.head_dim)
    kv, q, cents = g.kv, g.q, g.cents
    B, Hq, D = x.q.shape
    Hkv = x.k_cache.shape[1]
    cap = kv.select_capacity(budget)
    sel = torch.full((B, Hkv, cap), -1, dtype=torch.int32, device="cuda")
    cnt = torch.zeros((B, Hkv), dtype=torch.int32, device="cuda")
    out = torch.empty((B, Hq, D), dtype=A.torch_dtype(x.dtype), device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    ws_b = A.workspace(kv.workspace_bytes(budget, A.ABS_OP_BUILD))
    ws_s = A.workspace(kv.workspace_bytes(budget, A.ABS_OP_SELECT))
    ws_d = A.workspace(kv.workspace_bytes(budget, A.ABS_OP_DECODE))

    def step(st):
        A.build_centroids(kv, cents, ws=ws_b, stream=st)
        A.score_select(kv, cents, q, budget, sel, cnt, ws=ws_s, stream=st)
        A.sparse_decode(kv, q, sel, cnt, budget, sm, out, lse, ws=ws_d, stream=st)

    step(A.current_stream())
    torch.cuda.synchronize()
    want = [t.clone() for t in (cents.codes, sel, cnt, out.view(torch.int16) if dtype == "bf16" else out, lse)]
    ref_out, ref_lse = oracle_mod.attend(x.q, x.k_cache, x.v_cache, x.page_table, x.seq_lens, x.block_size,
                                         sel.cpu().numpy(), cnt.cpu().numpy(), sm, x.dtype)
    check_attention(out.float().cpu().numpy(), lse.cpu().numpy(), ref_out, ref_lse, x.dtype)

    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            step(int(side.cuda_stream))
    torch.cuda.synchronize()
    for rep in range(5):
        # eager work between replays: scramble the outputs
        sel.fill_(-7)
        cnt.fill_(0)
        out.zero_()
        lse.fill_(3.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        # selection slots past K are not written: compare the first K of each row
        kept = torch.arange(cap, device="cuda")[None, None, :] < want[2][:, :, None]
        got = (cents.codes, sel[kept], cnt, out.view(torch.int16) if dtype == "bf16" else out, lse)
        exp = (want[0], want[1][kept], want[2], want[3], want[4])
        for name, a, b in zip(("codes", "sel", "count", "out", "lse"), got, exp):
            assert torch.equal(a, b), (rep, name)
