"""Parity of abs_update_centroids (centroids kept current while decoding) with
the oracle, on the GPU, through the C ABI.

The caches hold every token up to L; the layer is built as if it had L0 =
L - appended tokens (centroid rows at capacity offsets), then updated to L.
Codes must be bit-exact (the update sums keys in fp64 like the build) and
the clamped-code counts exact.  Selection and attention then run on the
updated store (gapped centroid rows) and are compared under the usual rules.
"""
import numpy as np
import pytest
import torch

from block_sparse_attention_abs_amd import abs as A
from block_sparse_attention_abs_amd import workload as W
from gpu_pipeline import check_attention, check_selection, default_scale, unpack_codes

pytestmark = pytest.mark.gpu
P = W.PRESETS


def compact(codes, seq_lens, block_size, off):
    """Rows at offsets `off` -> compact CSR rows (the oracle's layout)."""
    out = []
    for i, (L, bs) in enumerate([(L, bs) for L in seq_lens for bs in block_size]):
        n = (int(L) + int(bs) - 1) // int(bs)
        out.append(codes[off[i]:off[i] + n])
    return np.concatenate(out, axis=0)


def spread(codes, seq_lens, block_size, off, D):
    out = np.zeros((int(off[-1]), D), dtype=np.uint8)
    r = 0
    for i, (L, bs) in enumerate([(L, bs) for L in seq_lens for bs in block_size]):
        n = (int(L) + int(bs) - 1) // int(bs)
        out[off[i]:off[i] + n] = codes[r:r + n]
        r += n
    return out


CASES = [
    ("bf16-d128", dict(), [4096, 3001], 1),
    ("bf16-d128", dict(), [4096, 3001], 16),
    ("bf16-d128", dict(), [4096, 3001], 17),
    ("bf16-d128", dict(), [4096, 3001], 100),
    ("bf16-d128", dict(), [4096, 3001], 0),
    ("f32-d64-g8", dict(dtype="f32", head_dim=64, num_q_heads=16, num_kv_heads=2), [2000, 1537], 33),
]


@pytest.mark.parametrize("name,kw,lens,appended", CASES)
def test_update_matches_oracle(oracle_mod, name, kw, lens, appended):
    w = P[1].scaled(batch=len(lens), context=max(lens), **kw)
    x = W.make_layer(w, seq_lens=lens)
    L = np.asarray(lens, dtype=np.int32)
    L0 = np.maximum(L - appended, 1).astype(np.int32)
    print(f"[gpu update] {name} lens={lens} appended={appended} bs={x.block_size.tolist()}", flush=True)
    cap = int(L.max())
    kv0 = A.PagedKV.from_host(x.q.shape[1], x.k_cache, x.v_cache, x.page_table, L0, x.block_size, x.dtype,
                              capacity_tokens=cap)
    cents = A.build_centroids(kv0, A.Centroids.empty(kv0))
    kv1 = kv0.with_lengths(L)
    oor = torch.full((len(lens), x.k_cache.shape[1]), -1, dtype=torch.int32, device="cuda")
    A.update_centroids(kv1, cents, appended, oor)
    torch.cuda.synchronize()
    off = kv0.centroid_off.cpu().numpy()
    D = x.k_cache.shape[3]

    c0 = oracle_mod.centroids(x.k_cache, x.page_table, L0, x.block_size, x.dtype)
    qz0 = oracle_mod.quantize(c0, L0, x.block_size)
    np.testing.assert_array_equal(cents.scale.cpu().numpy(), qz0.scale)
    np.testing.assert_array_equal(cents.lo.cpu().numpy(), qz0.lo)
    start = spread(qz0.codes, L0, x.block_size, off, D)
    want, want_oor = oracle_mod.update(x.k_cache, x.page_table, L, L0, x.block_size, off,
                                       oracle_mod.Quantized(start, qz0.scale, qz0.lo), x.dtype)
    got = unpack_codes(cents.codes.cpu().numpy())
    np.testing.assert_array_equal(got, want)
    np.testing.assert_array_equal(oor.cpu().numpy(), want_oor)

    # selection and attention on the updated store, whose rows have gaps
    budget = w.token_budget
    q = A.upload(x.q, "cuda", x.dtype)
    cap_sel = kv1.select_capacity(budget)
    sel = torch.full((len(lens), x.k_cache.shape[1], cap_sel), -1, dtype=torch.int32, device="cuda")
    cnt = torch.zeros((len(lens), x.k_cache.shape[1]), dtype=torch.int32, device="cuda")
    A.score_select(kv1, cents, q, budget, sel, cnt)
    sm = default_scale(D)
    out = torch.empty(tuple(x.q.shape), dtype=A.torch_dtype(x.dtype), device="cuda")
    lse = torch.empty(tuple(x.q.shape[:2]), dtype=torch.float32, device="cuda")
    A.sparse_decode(kv1, q, sel, cnt, budget, sm, out, lse)
    torch.cuda.synchronize()
    qz1 = oracle_mod.Quantized(compact(want, L, x.block_size, off), qz0.scale, qz0.lo)
    s1 = oracle_mod.scores(x.q, qz1, L, x.block_size, x.dtype)
    sel_h, cnt_h = sel.cpu().numpy(), cnt.cpu().numpy()
    check_selection(oracle_mod, x, qz1, s1, sel_h, cnt_h, budget)
    ref_out, ref_lse = oracle_mod.attend(x.q, x.k_cache, x.v_cache, x.page_table, L, x.block_size, sel_h, cnt_h,
                                         sm, x.dtype)
    check_attention(out.float().cpu().numpy(), lse.cpu().numpy(), ref_out, ref_lse, x.dtype)


@pytest.mark.parametrize("appended", [1, 17])
def test_update_full_size_sampled(oracle_mod, appended):
    """128K-token contexts, 4 sequences (the benchmark's workload): build at
    L - appended, update to L; the oracle recomputes the first and the last
    sequence on their own (bit-exact codes and clamp counts)."""
    w = P[3]
    x = W.make_layer(w, 0)
    L = x.seq_lens.astype(np.int32)
    L0 = (L - appended).astype(np.int32)
    Hkv, D = x.k_cache.shape[1], x.k_cache.shape[3]
    print(f"[gpu update] full size {w.name} appended={appended} bs={x.block_size.tolist()}", flush=True)
    kv0 = A.PagedKV.from_host(x.q.shape[1], x.k_cache, x.v_cache, x.page_table, L0, x.block_size, x.dtype,
                              capacity_tokens=int(L.max()))
    cents = A.build_centroids(kv0, A.Centroids.empty(kv0))
    oor = torch.full((len(L), Hkv), -1, dtype=torch.int32, device="cuda")
    A.update_centroids(kv0.with_lengths(L), cents, appended, oor)
    torch.cuda.synchronize()
    off = kv0.centroid_off.cpu().numpy()
    got = unpack_codes(cents.codes.cpu().numpy())
    got_oor = oor.cpu().numpy()
    for b in sorted({0, len(L) - 1}):
        pt = x.page_table[b:b + 1]
        c0 = oracle_mod.centroids(x.k_cache, pt, L0[b:b + 1], x.block_size, x.dtype)
        qz0 = oracle_mod.quantize(c0, L0[b:b + 1], x.block_size)
        off_b = off[b * Hkv:(b + 1) * Hkv + 1] - off[b * Hkv]
        start = spread(qz0.codes, L0[b:b + 1], x.block_size, off_b, D)
        want, want_oor = oracle_mod.update(x.k_cache, pt, L[b:b + 1], L0[b:b + 1], x.block_size, off_b,
                                           oracle_mod.Quantized(start, qz0.scale, qz0.lo), x.dtype)
        np.testing.assert_array_equal(got[off[b * Hkv]:off[(b + 1) * Hkv]], want)
        np.testing.assert_array_equal(got_oor[b], want_oor[0])
    del kv0, cents
    torch.cuda.empty_cache()
