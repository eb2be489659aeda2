"""abs_select_decode_static (no workspace argument: the library's per-GPU
static scratch) against abs_select_decode on a caller workspace, through
the C ABI: sel, sel_count, out and lse bit for bit, on two calls in a row,
the second with a smaller layer (the scratch keeps the first call's
contents), then the first layer again."""
import numpy as np
import pytest
import torch

from block_sparse_attention_abs_amd import abs as A
from block_sparse_attention_abs_amd import workload as W
from gpu_pipeline import GpuLayer, default_scale, to_host_f32

pytestmark = pytest.mark.gpu

P = W.PRESETS


def _run(g, budget, static):
    x = g.x
    B, Hq, D = x.q.shape
    Hkv = x.k_cache.shape[1]
    cap = g.kv.select_capacity(budget)
    sel = torch.full((B, Hkv, cap), -1, dtype=torch.int32, device="cuda")
    cnt = torch.zeros((B, Hkv), dtype=torch.int32, device="cuda")
    out = torch.full((B, Hq, D), 3.0, dtype=A.torch_dtype(x.dtype), device="cuda")
    lse = torch.full((B, Hq), 3.0, dtype=torch.float32, device="cuda")
    sm = default_scale(D)
    if static:
        A.abs_select_decode_static(g.kv.kv, g.kv.bmap, g.cents.desc, g.q.data_ptr(), budget, sm, sel.data_ptr(), cap,
                                   cnt.data_ptr(), out.data_ptr(), lse.data_ptr(), A.current_stream())
    else:
        A.select_decode(g.kv, g.cents, g.q, budget, sm, sel, cnt, out, lse)
    torch.cuda.synchronize()
    return sel.cpu().numpy(), cnt.cpu().numpy(), to_host_f32(out), lse.cpu().numpy()


def _equal(a, b):
    np.testing.assert_array_equal(a[1], b[1])
    for (bb, h), k in np.ndenumerate(a[1]):
        np.testing.assert_array_equal(a[0][bb, h, :k], b[0][bb, h, :k])
    np.testing.assert_array_equal(a[2], b[2])
    np.testing.assert_array_equal(a[3], b[3])


def test_static_scratch_call_equals_workspace_call():
    big = W.make_layer(P[1].scaled(batch=3, context=16384, token_budget=2048), seq_lens=[16384, 9001, 300])
    small = W.make_layer(P[1].scaled(batch=2, context=3000, token_budget=512), seq_lens=[3000, 1234])
    layers = []
    for x in (big, small):
        g = GpuLayer(x)
        g.build()
        budget = x.workload.token_budget
        need = g.kv.workspace_bytes(budget, A.ABS_OP_SELECT_DECODE)
        assert need <= A.STATIC_SCRATCH_BYTES
        print(f"[gpu no-alloc] B={x.q.shape[0]} lens={x.seq_lens.tolist()} plan={g.kv.launch_plan(budget)} "
              f"scratch need {need} B", flush=True)
        layers.append((g, budget, _run(g, budget, static=False)))
    for g, budget, want in layers + layers[:1]:
        _equal(_run(g, budget, static=True), want)
