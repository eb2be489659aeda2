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


def test_plain_host_program_matches_binding(oracle_mod, tmp_path):
    """tests/c/decode_step (a C++ host program with no Python or torch:
    hipMalloc, the abs.h descriptors, build, select, decode) gives the same
    selection and bit-identical outputs as the binding on the same inputs,
    and the attention matches the oracle on that selection."""
    import os
    import subprocess
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    exe = os.path.join(root, "tests", "c", "decode_step")
    assert os.path.exists(exe), "tests/c/decode_step is missing: run __graft_entry__.build()"
    w = W.PRESETS[1].scaled(batch=3, num_q_heads=16, num_kv_heads=4, head_dim=64, context=3000, dtype="f32",
                            token_budget=512, fixed_block_sizes=(16, 64, 32, 16))
    x = W.make_layer(w, seq_lens=[3000, 1234, 77])
    print("[gpu host program] f32 d64 g4 lens=[3000, 1234, 77]", flush=True)
    for name, arr in (("k", x.k_cache), ("v", x.v_cache), ("q", x.q), ("pt", x.page_table), ("lens", x.seq_lens)):
        np.ascontiguousarray(arr).tofile(tmp_path / f"{name}.bin")
    B, Hq, D = x.q.shape
    Hkv = x.k_cache.shape[1]
    args = [exe, str(tmp_path), str(B), str(Hq), str(Hkv), str(D), str(x.page_table.shape[1]),
            str(x.k_cache.shape[0]), str(w.token_budget)] + [str(int(b)) for b in x.block_size]
    r = subprocess.run(args, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    cap = int(r.stdout.split()[1])
    sel_c = np.fromfile(tmp_path / "sel.bin", dtype=np.int32).reshape(B, Hkv, cap)
    cnt_c = np.fromfile(tmp_path / "count.bin", dtype=np.int32).reshape(B, Hkv)
    out_c = np.fromfile(tmp_path / "out.bin", dtype=np.float32).reshape(B, Hq, D)
    lse_c = np.fromfile(tmp_path / "lse.bin", dtype=np.float32).reshape(B, Hq)

    g = GpuLayer(x)
    res = g.run(w.token_budget, float(np.float32(1.0 / np.sqrt(D))))
    np.testing.assert_array_equal(cnt_c, res.count)
    for (b, h), k in np.ndenumerate(res.count):
        np.testing.assert_array_equal(sel_c[b, h, :k], res.sel[b, h, :k])
    np.testing.assert_array_equal(out_c, res.out)
    np.testing.assert_array_equal(lse_c, res.lse)
    sm = float(np.float32(1.0 / np.sqrt(D)))
    ref_out, ref_lse = oracle_mod.attend(x.q, x.k_cache, x.v_cache, x.page_table, x.seq_lens, x.block_size, sel_c,
                                         cnt_c, sm, x.dtype)
    check_attention(out_c, lse_c, ref_out, ref_lse, x.dtype)
