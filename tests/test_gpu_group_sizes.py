"""Query groups of 3, 5, 6 and 7 heads per KV head through the C ABI: the
kernels run group sizes up to 8 in slots of 1, 2, 4 or 8 heads, the unused
slots padded, so a group that does not fill its slots exercises that
padding in the query fold of the score launch and in the decode's rows.
Each case runs the separate calls against the oracle (codes bit for bit,
the selection under the tie-band rule, attention on the GPU's selection;
gpu_pipeline's rules) and abs_select_decode against the separate calls, bit
for bit (the larger G = 3 bf16 layer takes the fused launch)."""
import numpy as np
import pytest
import torch

from block_sparse_attention_abs_amd import abs as A
from block_sparse_attention_abs_amd import workload as W
from gpu_pipeline import check_attention, check_selection, codes_of_format, default_scale

pytestmark = pytest.mark.gpu

CASES = {
    # name: (G, Hkv, head_dim, dtype, lens, budget, block sizes)
    "g3-bf16-d128": (3, 4, 128, "bf16", [8192, 6000, 5000, 4500], 4096, (16, 64, 32, 64)),   # fused
    "g3-bf16-d128-small": (3, 2, 128, "bf16", [6000, 2501], 1024, (16, 64)),   # separate launches
    "g3-f32-d64": (3, 3, 64, "f32", [3001, 999], 512, (32, 16, 64)),
    "g5-bf16-d128": (5, 2, 128, "bf16", [4000, 77], 512, (64, 16)),
    "g6-bf16-d64": (6, 2, 64, "bf16", [5000, 1234], 1024, (16, 32)),
    "g7-f32-d128": (7, 1, 128, "f32", [2500, 2049], 512, (32,)),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_group_size(oracle_mod, name):
    G, Hkv, D, dtype, lens, budget, bs = CASES[name]
    w = W.PRESETS[1].scaled(batch=len(lens), num_q_heads=G * Hkv, num_kv_heads=Hkv, head_dim=D, dtype=dtype,
                            context=max(lens), token_budget=budget, fixed_block_sizes=bs)
    x = W.make_layer(w, seq_lens=lens)
    B, Hq, _ = x.q.shape
    print(f"[gpu groups] {name}: G={G} Hkv={Hkv} D={D} {dtype} lens={lens} bs={list(bs)} budget={budget}",
          flush=True)
    kv = A.PagedKV.from_host(Hq, x.k_cache, x.v_cache, x.page_table, x.seq_lens, x.block_size, x.dtype)
    cents = A.build_centroids(kv, A.Centroids.empty(kv))
    q = A.upload(x.q, "cuda", x.dtype)
    sm = default_scale(D)
    cap = kv.select_capacity(budget)

    def buffers():
        return (torch.full((B, Hkv, cap), -1, dtype=torch.int32, device="cuda"),
                torch.zeros((B, Hkv), dtype=torch.int32, device="cuda"),
                torch.empty((B, Hq, D), dtype=A.torch_dtype(x.dtype), device="cuda"),
                torch.empty((B, Hq), dtype=torch.float32, device="cuda"))

    sel, cnt, out, lse = buffers()
    A.score_select(kv, cents, q, budget, sel, cnt)
    A.sparse_decode(kv, q, sel, cnt, budget, sm, out, lse)
    fsel, fcnt, fout, flse = buffers()
    A.select_decode(kv, cents, q, budget, sm, fsel, fcnt, fout, flse)
    torch.cuda.synchronize()
    if name == "g3-bf16-d128" and kv.launch_plan(budget)["compute_units"] == 256:
        assert kv.launch_plan(budget)["fused"] == 1

    sel_h, cnt_h = sel.cpu().numpy(), cnt.cpu().numpy()
    np.testing.assert_array_equal(fcnt.cpu().numpy(), cnt_h)
    fsel_h = fsel.cpu().numpy()
    for (b, h), k in np.ndenumerate(cnt_h):
        np.testing.assert_array_equal(fsel_h[b, h, :k], sel_h[b, h, :k])
    np.testing.assert_array_equal(fout.float().cpu().numpy(), out.float().cpu().numpy())
    np.testing.assert_array_equal(flse.cpu().numpy(), lse.cpu().numpy())

    c = oracle_mod.centroids(x.k_cache, x.page_table, x.seq_lens, x.block_size, x.dtype)
    qf = oracle_mod.quantize_fmt(c, x.seq_lens, x.block_size, "int4")
    np.testing.assert_array_equal(codes_of_format(cents.codes.cpu().numpy(), "int4"), qf.codes)
    s = oracle_mod.scores_dense(x.q, qf.deq, x.seq_lens, x.block_size, x.dtype)
    check_selection(oracle_mod, x, qf, s, sel_h, cnt_h, budget)
    ref_out, ref_lse = oracle_mod.attend(x.q, x.k_cache, x.v_cache, x.page_table, x.seq_lens, x.block_size, sel_h,
                                         cnt_h, sm, x.dtype)
    check_attention(out.float().cpu().numpy(), lse.cpu().numpy(), ref_out, ref_lse, x.dtype)
