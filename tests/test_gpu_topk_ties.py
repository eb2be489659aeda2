"""Top-K with runs of equal scores at the threshold, through the C ABI against
the oracle.

Blocks whose 16 keys all equal one vector v have equal centroids, equal codes
and so equal scores.  With v = a * sign(qbar) (qbar the head's group query
sum) every channel's weight qbar_d * scale_d meets v's code at the same side
of the range, so a = 10 scores above a = 5, which scores above the Gaussian
blocks.  Sizes of the two groups put the K-th largest score into a histogram
bin with a few candidates, into a crowded bin, or into a bin with more
candidates than the top-K kernel's candidate list holds (where it falls back
to a radix select over the keys).  Ties go to the lower block index (the
selection rule of the oracle), so the expected set is known exactly: the
a = 10 group, then the lowest-indexed blocks of the a = 5 group.
"""
import numpy as np
import pytest

from block_sparse_attention_abs_amd import workload as W
from gpu_pipeline import GpuLayer, check_attention, check_selection, default_scale

pytestmark = pytest.mark.gpu

#       name          context  K   |a=10|  |a=5|
CASES = [("few-below", 4096, 32, 10, 50),     # threshold bin = the a=5 group: 50 candidates, 22 kept
         ("few-all", 4096, 32, 0, 40),        # every kept block is a candidate
         ("edge-64", 4096, 32, 10, 64),       # 64 candidates: the most one wavefront ranks
         ("edge-65", 4096, 32, 10, 65),       # 65: ranked through LDS by the candidates' threads
         ("crowded", 4096, 32, 10, 200),      # 200 candidates
         ("overflow", 16384, 32, 0, 600),     # more than the candidate list holds: radix select
         # 4096 blocks per head (8 keys per thread): the same three paths
         ("wide-few", 65536, 32, 10, 50),
         ("wide-crowded", 65536, 32, 10, 200),
         ("wide-overflow", 65536, 32, 0, 600)]


def _layer(context, K, n10, n5, dtype, seed):
    w = W.PRESETS[1].scaled(batch=2, context=context, dtype=dtype, token_budget=16 * K,
                            fixed_block_sizes=(16,) * 8)
    lens = [context, context - 100]
    x = W.make_layer(w, seq_lens=lens, needles=False)
    rng = np.random.default_rng(seed)
    qf = W.to_f32(x.q, dtype).astype(np.float64)
    G = w.num_q_heads // w.num_kv_heads
    groups = {}
    for b, L in enumerate(lens):
        N = -(-L // 16)
        for h in range(w.num_kv_heads):
            sign = np.sign(qf[b, h * G:(h + 1) * G].sum(axis=0))
            assert (sign != 0).all()
            pick = rng.permutation(N)
            s10, s5 = np.sort(pick[:n10]), np.sort(pick[n10:n10 + n5])
            for blocks, a in ((s10, 10.0), (s5, 5.0)):
                v = W.to_storage((a * sign).astype(np.float32)[None, :].repeat(16, axis=0), dtype)
                for j in blocks:
                    x.k_cache[x.page_table[b, j], h] = v
            groups[(b, h)] = (s10, s5)
    return x, groups


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("name,context,K,n10,n5", CASES)
def test_threshold_ties(oracle_mod, name, context, K, n10, n5, dtype):
    x, groups = _layer(context, K, n10, n5, dtype, seed=context + n5)
    budget = 16 * K
    print(f"[gpu topk ties] {name} {dtype}: context {context}, K {K}, groups {n10}/{n5}", flush=True)
    sm = default_scale(x.q.shape[2])
    r = GpuLayer(x).run(budget, sm)
    ref = oracle_mod.run(x, sm_scale=sm, budget=budget)
    np.testing.assert_array_equal(r.codes, ref.quant.codes)
    check_selection(oracle_mod, x, ref.quant, ref.scores, r.sel, r.count, budget)
    Hkv = x.k_cache.shape[1]
    row = 0
    for b, L in enumerate(x.seq_lens.tolist()):
        N = -(-L // 16)
        for h in range(Hkv):
            s10, s5 = groups[(b, h)]
            sc = ref.scores[row:row + N]
            rest = np.setdiff1d(np.arange(N), np.concatenate([s10, s5]))
            # the construction's ordering, on the oracle's own scores
            assert len(np.unique(sc[s5])) == 1 and sc[s5].min() > sc[rest].max()
            if len(s10):
                assert len(np.unique(sc[s10])) == 1 and sc[s10].min() > sc[s5].max()
            if name.startswith("edge"):
                # the a = 5 group alone fills the threshold bin: every other
                # score lies more than two of the 2048 bin widths below it
                assert sc[s5].min() - sc[rest].max() > 2 * (sc.max() - sc.min()) / 2048
            want = np.sort(np.concatenate([s10, s5[:K - len(s10)]]))
            assert r.count[b, h] == K
            np.testing.assert_array_equal(r.sel[b, h, :K], want)
            row += N
    out, lse = oracle_mod.attend(x.q, x.k_cache, x.v_cache, x.page_table, x.seq_lens, x.block_size, r.sel, r.count,
                                 sm, x.dtype)
    check_attention(r.out, r.lse, out, lse, x.dtype)
