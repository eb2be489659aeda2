"""Parity of the centroid storage formats (the precisions Figure 8 of the
AB-Sparse page compares: INT4 asymmetric per channel, INT4 symmetric, INT8,
INT4 with one range per head, bf16) with the oracle, on the GPU, through the
C ABI.

Per format: codes, scale and lo are bit-exact (the kernels take the same
fp32 steps as the oracle's definitions, after the same correctly rounded
fp32 mean); the selection follows the rules of gpu_pipeline.py against the
oracle's fp64 scores of the dequantized centroids; the update after appends
(with keys far outside the built range, so codes clamp) is bit-exact with
exact clamp counts.
"""
import dataclasses

import numpy as np
import pytest
import torch

from block_sparse_attention_abs_amd import abs as A
from block_sparse_attention_abs_amd import workload as W
from gpu_pipeline import check_attention, check_selection, codes_of_format, default_scale

pytestmark = pytest.mark.gpu
P = W.PRESETS
FORMATS = ["int4", "int4_sym", "int8", "int4_tensor", "bf16"]
CASES = {
    "llama-4k-ragged": (dict(batch=2, context=4096, token_budget=512), [4096, 3001]),
    "gqa8-d64-f32": (dict(num_q_heads=16, num_kv_heads=2, head_dim=64, dtype="f32", context=3000, token_budget=512,
                          batch=2), [3000, 2222]),
}


def _select(kv, cents, q, budget, B, Hkv):
    cap = kv.select_capacity(budget)
    sel = torch.full((B, Hkv, cap), -1, dtype=torch.int32, device="cuda")
    cnt = torch.zeros((B, Hkv), dtype=torch.int32, device="cuda")
    A.score_select(kv, cents, q, budget, sel, cnt)
    return sel, cnt


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("case", list(CASES))
def test_format_build_select_decode(oracle_mod, case, fmt):
    kw, lens = CASES[case]
    w = P[1].scaled(**kw)
    x = W.make_layer(w, seq_lens=lens)
    B, Hq, D = x.q.shape
    Hkv = x.k_cache.shape[1]
    print(f"[gpu formats] {case} {fmt} lens={lens} bs={x.block_size.tolist()}", flush=True)
    kv = A.PagedKV.from_host(Hq, x.k_cache, x.v_cache, x.page_table, x.seq_lens, x.block_size, x.dtype)
    cents = A.build_centroids(kv, A.Centroids.empty(kv, fmt))
    q = A.upload(x.q, "cuda", x.dtype)
    sel, cnt = _select(kv, cents, q, w.token_budget, B, Hkv)
    sm = default_scale(D)
    out = torch.empty((B, Hq, D), dtype=A.torch_dtype(x.dtype), device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    A.sparse_decode(kv, q, sel, cnt, w.token_budget, sm, out, lse)
    torch.cuda.synchronize()

    c = oracle_mod.centroids(x.k_cache, x.page_table, x.seq_lens, x.block_size, x.dtype)
    qf = oracle_mod.quantize_fmt(c, x.seq_lens, x.block_size, fmt)
    np.testing.assert_array_equal(codes_of_format(cents.codes.cpu().numpy(), fmt), qf.codes)
    np.testing.assert_array_equal(cents.scale.cpu().numpy(), qf.scale)
    np.testing.assert_array_equal(cents.lo.cpu().numpy(), qf.lo)
    s = oracle_mod.scores_dense(x.q, qf.deq, x.seq_lens, x.block_size, x.dtype)
    sel_h, cnt_h = sel.cpu().numpy(), cnt.cpu().numpy()
    check_selection(oracle_mod, x, qf, s, sel_h, cnt_h, w.token_budget)
    ref_out, ref_lse = oracle_mod.attend(x.q, x.k_cache, x.v_cache, x.page_table, x.seq_lens, x.block_size, sel_h,
                                         cnt_h, sm, x.dtype)
    check_attention(out.float().cpu().numpy(), lse.cpu().numpy(), ref_out, ref_lse, x.dtype)


def _spread(codes, seq_lens, block_size, off):
    out = np.zeros((int(off[-1]), codes.shape[1]), dtype=codes.dtype)
    r = 0
    for i, (L, bs) in enumerate([(L, bs) for L in seq_lens for bs in block_size]):
        n = (int(L) + int(bs) - 1) // int(bs)
        out[off[i]:off[i] + n] = codes[r:r + n]
        r += n
    return out


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("dtype,appended,far", [("bf16", 17, False), ("f32", 33, True)])
def test_format_update(oracle_mod, fmt, dtype, appended, far):
    """Build at L - appended (rows at capacity offsets), update to L; far: the
    appended keys are 1000 (outside every built range; bf16 holds it)."""
    lens = [4096, 3001]
    w = P[1].scaled(batch=2, context=max(lens), dtype=dtype)
    x = W.make_layer(w, seq_lens=lens)
    L = np.asarray(lens, dtype=np.int32)
    L0 = (L - appended).astype(np.int32)
    if far:
        assert dtype == "f32"
        for b in range(len(lens)):
            for t in range(int(L0[b]), int(L[b])):
                x.k_cache[x.page_table[b, t // 16], :, t % 16, :] = np.float32(1e3)
    print(f"[gpu formats] update {fmt} {dtype} appended={appended} far={far}", flush=True)
    kv0 = A.PagedKV.from_host(x.q.shape[1], x.k_cache, x.v_cache, x.page_table, L0, x.block_size, x.dtype,
                              capacity_tokens=int(L.max()))
    cents = A.build_centroids(kv0, A.Centroids.empty(kv0, fmt))
    kv1 = kv0.with_lengths(L)
    oor = torch.full((len(lens), x.k_cache.shape[1]), -1, dtype=torch.int32, device="cuda")
    A.update_centroids(kv1, cents, appended, oor)
    torch.cuda.synchronize()
    off = kv0.centroid_off.cpu().numpy()

    c0 = oracle_mod.centroids(x.k_cache, x.page_table, L0, x.block_size, x.dtype)
    qf = oracle_mod.quantize_fmt(c0, L0, x.block_size, fmt)
    np.testing.assert_array_equal(cents.scale.cpu().numpy(), qf.scale)
    np.testing.assert_array_equal(cents.lo.cpu().numpy(), qf.lo)
    start = _spread(qf.codes, L0, x.block_size, off)
    want, want_oor = oracle_mod.update(x.k_cache, x.page_table, L, L0, x.block_size, off,
                                       dataclasses.replace(qf, codes=start), x.dtype, fmt)
    np.testing.assert_array_equal(codes_of_format(cents.codes.cpu().numpy(), fmt), want)
    np.testing.assert_array_equal(oor.cpu().numpy(), want_oor)
    if far:
        assert (want_oor == 0).all() if fmt == "bf16" else (want_oor > 0).all()


@pytest.mark.parametrize("fmt", ["int4_sym", "int8", "int4_tensor", "bf16"])
def test_format_full_size_sampled(oracle_mod, fmt):
    """128K-token contexts, 4 sequences (the benchmark's workload), every
    format: the oracle recomputes the first and the last sequence."""
    w = P[3]
    x = W.make_layer(w, 0)
    print(f"[gpu formats] full size {w.name} {fmt} bs={x.block_size.tolist()}", flush=True)
    B, Hq, D = x.q.shape
    Hkv = x.k_cache.shape[1]
    kv = A.PagedKV.from_host(Hq, x.k_cache, x.v_cache, x.page_table, x.seq_lens, x.block_size, x.dtype)
    cents = A.build_centroids(kv, A.Centroids.empty(kv, fmt))
    q = A.upload(x.q, "cuda", x.dtype)
    sel, cnt = _select(kv, cents, q, w.token_budget, B, Hkv)
    torch.cuda.synchronize()
    codes = codes_of_format(cents.codes.cpu().numpy(), fmt)
    scale, lo = cents.scale.cpu().numpy(), cents.lo.cpu().numpy()
    sel_h, cnt_h = sel.cpu().numpy(), cnt.cpu().numpy()
    off = kv.centroid_off.cpu().numpy()
    for b in sorted({0, B - 1}):
        xb = dataclasses.replace(x, q=x.q[b:b + 1], page_table=x.page_table[b:b + 1], seq_lens=x.seq_lens[b:b + 1])
        c = oracle_mod.centroids(x.k_cache, xb.page_table, xb.seq_lens, x.block_size, x.dtype)
        qf = oracle_mod.quantize_fmt(c, xb.seq_lens, x.block_size, fmt)
        np.testing.assert_array_equal(codes[off[b * Hkv]:off[(b + 1) * Hkv]], qf.codes)
        np.testing.assert_array_equal(scale[b], qf.scale[0])
        np.testing.assert_array_equal(lo[b], qf.lo[0])
        s = oracle_mod.scores_dense(xb.q, qf.deq, xb.seq_lens, x.block_size, x.dtype)
        check_selection(oracle_mod, xb, qf, s, sel_h[b:b + 1], cnt_h[b:b + 1], w.token_budget)
    del kv, cents
    torch.cuda.empty_cache()
