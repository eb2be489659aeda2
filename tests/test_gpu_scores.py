"""The score launch's values, not only the selection made from them, against
the oracle's fp64 scores on the same centroid codes.

abs_estimate leaves the score rows at the start of the select region of its
workspace: fp32, one row per (b, h) in b-major order, each row as long as
the layer's largest block count rounded up to a multiple of 4.  For 4- and
8-bit codes the kernel sums code x weight exactly in integers after rounding
each weight to a 30-bit integer multiple of a power of two (at most 2^-30 of
the largest weight of its run of 32 or 16 channels off), so a score is at
most 128 x (2^bits - 1) x 2^-30 max_d |w_d| <= 2.4e-7 M off before it is
stored, M = sum_d |qbar_d| max(|lo_d|, |hi_d|) >= (2^bits - 1) max_d |w_d| / 2
(R16's bound on every |score|); bf16 centroids are summed in fp64.  Storing
the row in fp32 adds half an ulp.  The bound checked: |gpu - oracle| <=
2.4e-7 M + 2^-24 |oracle| + 1e-12 M.
"""
import numpy as np
import pytest
import torch

from block_sparse_attention_abs_amd import abs as A
from block_sparse_attention_abs_amd import workload as W
from gpu_pipeline import codes_of_format

pytestmark = pytest.mark.gpu

LEVELS = {"int4": 15, "int4_sym": 15, "int4_tensor": 15, "int8": 255}


def _layer(name):
    if name == "b2-8k":
        return W.make_layer(W.PRESETS[1].scaled(batch=2, context=8192), seq_lens=[8192, 3001])
    if name == "d64-gqa2-f32":
        return W.make_layer(W.PRESETS[1].scaled(batch=2, num_q_heads=8, num_kv_heads=4, head_dim=64, dtype="f32",
                                                context=5000), seq_lens=[5000, 77])
    raise KeyError(name)


@pytest.mark.parametrize("name,fmt", [("b2-8k", "int4"), ("b2-8k", "int4_sym"), ("b2-8k", "int4_tensor"),
                                      ("b2-8k", "int8"), ("b2-8k", "bf16"), ("d64-gqa2-f32", "int4")])
def test_score_values_within_the_arithmetic_bound(oracle_mod, name, fmt):
    x = _layer(name)
    B, Hq, D = x.q.shape
    Hkv = x.k_cache.shape[1]
    G = Hq // Hkv
    budget = x.workload.token_budget
    print(f"[gpu scores] {name} {fmt}: lens={x.seq_lens.tolist()} bs={x.block_size.tolist()}", flush=True)
    kv = A.PagedKV.from_host(Hq, x.k_cache, x.v_cache, x.page_table, x.seq_lens, x.block_size, x.dtype)
    cents = A.build_centroids(kv, A.Centroids.empty(kv, fmt))
    q = A.upload(x.q, "cuda", x.dtype)
    ws = A.workspace(kv.workspace_bytes(budget, A.ABS_OP_SELECT_DECODE))
    A.abs_estimate(kv.kv, kv.bmap, cents.desc, int(q.data_ptr()), budget, int(ws.data_ptr()), ws.numel(),
                   A.current_stream())
    torch.cuda.synchronize()
    stride = (kv.launch_plan(budget)["max_blocks"] + 3) // 4 * 4
    rows = ws[:B * Hkv * stride * 4].view(torch.float32).reshape(B * Hkv, stride).cpu().numpy()

    c = oracle_mod.centroids(x.k_cache, x.page_table, x.seq_lens, x.block_size, x.dtype)
    qf = oracle_mod.quantize_fmt(c, x.seq_lens, x.block_size, fmt)
    np.testing.assert_array_equal(codes_of_format(cents.codes.cpu().numpy(), fmt), qf.codes)
    s = oracle_mod.scores_dense(x.q, qf.deq, x.seq_lens, x.block_size, x.dtype)
    qfull = W.to_f32(x.q, x.dtype).astype(np.float64)
    worst = 0.0
    for b, h, r0, n in oracle_mod.block_rows(x.seq_lens, x.block_size):
        qbar = qfull[b, h * G:(h + 1) * G].sum(0)
        if fmt in LEVELS:
            lo = qf.lo[b, h].astype(np.float64)
            hi = lo + LEVELS[fmt] * qf.scale[b, h].astype(np.float64)
            M = float(np.sum(np.abs(qbar) * np.maximum(np.abs(lo), np.abs(hi))))
        else:
            M = float(np.sum(np.abs(qbar) * np.abs(qf.deq[r0:r0 + n]).max(axis=0)))
        got = rows[b * Hkv + h, :n].astype(np.float64)
        want = s[r0:r0 + n]
        bound = 2.4e-7 * M + 2.0 ** -24 * np.abs(want) + 1e-12 * M
        err = np.abs(got - want)
        assert (err <= bound).all(), (b, h, float(err.max()), float(bound.min()), M)
        worst = max(worst, float((err / (bound + 1e-300)).max()))
    print(f"[gpu scores] {name} {fmt}: largest error / bound {worst:.3f}", flush=True)
