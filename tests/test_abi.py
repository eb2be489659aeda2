"""The C ABI without a GPU: libabs.so loads, exports every call include/abs.h
declares, the Python structures match the C layouts, the host-side geometry
helpers agree with the oracle's block counts, and invalid descriptors are
rejected with the documented status before anything is enqueued."""
import ctypes as C
import os
import re
import subprocess

import numpy as np
import pytest

from block_sparse_attention_abs_amd import abs as A

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "abs.h")

pytestmark = pytest.mark.skipif(not os.path.exists(A.LIB_PATH), reason="libabs.so not built")


def header_functions():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(abs_\w+)\s*\(", txt, re.M)))


def test_exports_every_declared_call():
    names = header_functions()
    assert len(names) == 22
    assert sorted(A.EXPORTS) == names
    L = A.lib()
    for n in names:
        assert getattr(L, n) is not None
    out = subprocess.run(["nm", "-D", "--defined-only", A.LIB_PATH], capture_output=True, text=True, check=True)
    exported = set(re.findall(r" T (abs_\w+)", out.stdout))
    assert set(names) <= exported


def test_struct_layout_matches_c(tmp_path):
    src = tmp_path / "layout.c"
    src.write_text("""
#include <stdio.h>
#include <stddef.h>
#include "abs.h"
#define F(s, f) printf(#s "." #f " %zu\\n", offsetof(s, f))
int main(void) {
  printf("abs_paged_kv %zu\\nabs_block_map %zu\\nabs_centroids %zu\\n",
         sizeof(abs_paged_kv), sizeof(abs_block_map), sizeof(abs_centroids));
  F(abs_paged_kv, num_pages); F(abs_paged_kv, kv_dtype); F(abs_paged_kv, k_cache);
  F(abs_paged_kv, seq_lens_host); F(abs_block_map, centroid_off); F(abs_centroids, lo);
  F(abs_centroids, format); F(abs_centroids, reserved0);
  return 0;
}""")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = dict(l.split() for l in subprocess.run([str(exe)], capture_output=True, text=True).stdout.splitlines())
    assert int(got["abs_paged_kv"]) == C.sizeof(A.abs_paged_kv)
    assert int(got["abs_block_map"]) == C.sizeof(A.abs_block_map)
    assert int(got["abs_centroids"]) == C.sizeof(A.abs_centroids)
    for key, (st, f) in {"abs_paged_kv.num_pages": (A.abs_paged_kv, "num_pages"),
                         "abs_paged_kv.kv_dtype": (A.abs_paged_kv, "kv_dtype"),
                         "abs_paged_kv.k_cache": (A.abs_paged_kv, "k_cache"),
                         "abs_paged_kv.seq_lens_host": (A.abs_paged_kv, "seq_lens_host"),
                         "abs_block_map.centroid_off": (A.abs_block_map, "centroid_off"),
                         "abs_centroids.lo": (A.abs_centroids, "lo"),
                         "abs_centroids.format": (A.abs_centroids, "format"),
                         "abs_centroids.reserved0": (A.abs_centroids, "reserved0")}.items():
        assert int(got[key]) == getattr(st, f).offset


FAKE = 1 << 40  # stands in for a device address; never dereferenced on these paths


class Host:
    """Descriptors with host metadata and placeholder device pointers."""

    def __init__(self, seq_lens=(300, 77), block_size=(16, 64), Hq=4, D=64, dtype=A.ABS_BF16, max_pages=32):
        self.sl = np.asarray(seq_lens, dtype=np.int32)
        self.bs = np.asarray(block_size, dtype=np.int32)
        self.kv = A.abs_paged_kv(num_seqs=len(self.sl), num_q_heads=Hq, num_kv_heads=len(self.bs), head_dim=D,
                                 page_size=16, max_pages_per_seq=max_pages, num_pages=64, kv_dtype=dtype,
                                 reserved0=0, k_cache=FAKE, v_cache=FAKE, page_table=FAKE, seq_lens=FAKE,
                                 seq_lens_host=self.sl.ctypes.data)
        self.bmap = A.abs_block_map(block_size_host=self.bs.ctypes.data, block_size=FAKE, centroid_off=FAKE)
        self.cents = A.abs_centroids(codes=FAKE, scale=FAKE, lo=FAKE)


def test_geometry_helpers_agree_with_oracle(oracle_mod):
    h = Host(seq_lens=(300, 77, 1), block_size=(16, 64, 32), Hq=6)
    assert A.abs_total_blocks(h.kv, h.bmap) == oracle_mod.total_blocks(h.sl, h.bs)
    off = A.abs_centroid_offsets(h.kv, h.bmap)
    rows = oracle_mod.block_rows(h.sl, h.bs)
    assert off[:-1].tolist() == [r[2] for r in rows] and off[-1] == oracle_mod.total_blocks(h.sl, h.bs)
    for budget in (1, 17, 64, 100, 4096):
        assert A.abs_select_capacity(h.kv, h.bmap, budget) == oracle_mod.sel_capacity(h.sl, h.bs, budget)
    for op in (A.ABS_OP_BUILD, A.ABS_OP_SELECT, A.ABS_OP_DECODE, A.ABS_OP_SELECT_DECODE):
        assert A.abs_workspace_bytes(h.kv, h.bmap, 64, op) > 0
    # the fused call's workspace: the select workspace, then the decode workspace
    assert A.abs_workspace_bytes(h.kv, h.bmap, 64, A.ABS_OP_SELECT_DECODE) == (
        A.abs_workspace_bytes(h.kv, h.bmap, 64, A.ABS_OP_SELECT) + A.abs_workspace_bytes(h.kv, h.bmap, 64,
                                                                                          A.ABS_OP_DECODE))
    cap = A.abs_centroid_offsets_capacity(h.kv, h.bmap, 400)
    np.testing.assert_array_equal(cap, oracle_mod.csr_offsets(h.sl, h.bs, capacity_tokens=400))
    assert status_of(lambda: A.abs_centroid_offsets_capacity(h.kv, h.bmap, 299)) == A.ABS_ERR_INVALID_ARG


def status_of(fn):
    try:
        fn()
    except A.AbsError as e:
        assert A.abs_last_error()
        return e.status
    return A.ABS_OK


@pytest.mark.parametrize("field,value,want", [
    ("num_seqs", 0, A.ABS_ERR_INVALID_ARG),
    ("num_q_heads", 3, A.ABS_ERR_INVALID_ARG),
    ("num_q_heads", 36, A.ABS_ERR_UNSUPPORTED),
    ("head_dim", 96, A.ABS_ERR_UNSUPPORTED),
    ("page_size", 32, A.ABS_ERR_UNSUPPORTED),
    ("kv_dtype", 7, A.ABS_ERR_UNSUPPORTED),
    ("reserved0", 1, A.ABS_ERR_INVALID_ARG),
    ("max_pages_per_seq", 0, A.ABS_ERR_INVALID_ARG),
    ("max_pages_per_seq", 4, A.ABS_ERR_INVALID_ARG),      # 300 tokens do not fit in 4 pages
    ("seq_lens_host", None, A.ABS_ERR_INVALID_ARG),
])
def test_descriptor_validation(field, value, want):
    h = Host()
    setattr(h.kv, field, value)
    assert status_of(lambda: A.abs_total_blocks(h.kv, h.bmap)) == want
    assert status_of(lambda: A.abs_build_centroids(h.kv, h.bmap, h.cents, FAKE, 1 << 30, 0)) == want
    assert status_of(lambda: A.abs_update_centroids(h.kv, h.bmap, h.cents, 1, None, 0)) == want


@pytest.mark.parametrize("sizes,lens,want", [
    ((16, 48), (300, 77), A.ABS_ERR_UNSUPPORTED),
    ((16, 0), (300, 77), A.ABS_ERR_INVALID_ARG),
    ((16, 1), (300, 77), A.ABS_ERR_UNSUPPORTED),           # block size 1 exists in the oracle only
    ((16, 64), (0, 77), A.ABS_ERR_INVALID_ARG),
])
def test_block_map_and_length_validation(sizes, lens, want):
    h = Host(seq_lens=lens, block_size=sizes)
    assert status_of(lambda: A.abs_total_blocks(h.kv, h.bmap)) == want


def test_call_level_validation():
    h = Host()
    need_b = A.abs_workspace_bytes(h.kv, h.bmap, 64, A.ABS_OP_BUILD)
    need_s = A.abs_workspace_bytes(h.kv, h.bmap, 64, A.ABS_OP_SELECT)
    need_d = A.abs_workspace_bytes(h.kv, h.bmap, 64, A.ABS_OP_DECODE)
    cap = A.abs_select_capacity(h.kv, h.bmap, 64)
    W = A.ABS_ERR_WORKSPACE
    assert status_of(lambda: A.abs_build_centroids(h.kv, h.bmap, h.cents, FAKE, need_b - 1, 0)) == W
    assert status_of(lambda: A.abs_score_select(h.kv, h.bmap, h.cents, FAKE, 64, FAKE, cap, FAKE, FAKE,
                                                need_s - 1, 0)) == W
    assert status_of(lambda: A.abs_sparse_decode(h.kv, h.bmap, FAKE, FAKE, cap, FAKE, 64, 0.125, FAKE, None,
                                                 FAKE, need_d - 1, 0)) == W
    I = A.ABS_ERR_INVALID_ARG
    assert status_of(lambda: A.abs_score_select(h.kv, h.bmap, h.cents, FAKE, 64, FAKE, cap - 1, FAKE, FAKE,
                                                need_s, 0)) == I
    assert status_of(lambda: A.abs_score_select(h.kv, h.bmap, h.cents, FAKE, 0, FAKE, cap, FAKE, FAKE,
                                                need_s, 0)) == I
    assert status_of(lambda: A.abs_score_select(h.kv, h.bmap, h.cents, None, 64, FAKE, cap, FAKE, FAKE,
                                                need_s, 0)) == I
    assert status_of(lambda: A.abs_sparse_decode(h.kv, h.bmap, FAKE, FAKE, cap, FAKE, 64, float("nan"), FAKE,
                                                 None, FAKE, need_d, 0)) == I
    need_sd = A.abs_workspace_bytes(h.kv, h.bmap, 64, A.ABS_OP_SELECT_DECODE)
    assert status_of(lambda: A.abs_select_decode(h.kv, h.bmap, h.cents, FAKE, 64, 0.125, FAKE, cap, FAKE, FAKE,
                                                 None, FAKE, need_sd - 1, 0)) == W
    assert status_of(lambda: A.abs_select_decode(h.kv, h.bmap, h.cents, FAKE, 64, 0.125, FAKE, cap - 1, FAKE,
                                                 FAKE, None, FAKE, need_sd, 0)) == I
    assert status_of(lambda: A.abs_select_decode(h.kv, h.bmap, h.cents, FAKE, 64, 0.125, FAKE, cap, FAKE, None,
                                                 None, FAKE, need_sd, 0)) == I
    assert status_of(lambda: A.abs_select_decode(h.kv, h.bmap, h.cents, FAKE, 64, float("inf"), FAKE, cap, FAKE,
                                                 FAKE, None, FAKE, need_sd, 0)) == I
    assert status_of(lambda: A.abs_select_decode(h.kv, h.bmap, h.cents, None, 64, 0.125, FAKE, cap, FAKE, FAKE,
                                                 None, FAKE, need_sd, 0)) == I
    assert status_of(lambda: A.abs_update_centroids(h.kv, h.bmap, h.cents, -1, None, 0)) == I
    assert status_of(lambda: A.abs_update_centroids(h.kv, h.bmap, A.abs_centroids(codes=FAKE, scale=None, lo=FAKE),
                                                    1, None, 0)) == I
    h.kv.v_cache = None
    assert status_of(lambda: A.abs_sparse_decode(h.kv, h.bmap, FAKE, FAKE, cap, FAKE, 64, 0.125, FAKE, None,
                                                 FAKE, need_d, 0)) == I


@pytest.mark.parametrize("fmt,D,want", [(0, 128, 64), (1, 128, 64), (2, 128, 128), (3, 64, 32), (4, 64, 128),
                                        (4, 128, 256)])
def test_centroid_row_bytes(fmt, D, want):
    assert A.abs_centroid_row_bytes(D, fmt) == want
    assert A.CENTROID_FORMATS[["int4", "int4_sym", "int8", "int4_tensor", "bf16"][fmt]] == fmt


def test_centroid_format_validation():
    """Unknown formats, a non-zero reserved field and misaligned codes are
    rejected by every call that takes a centroid store."""
    assert status_of(lambda: A.abs_centroid_row_bytes(64, 5)) == A.ABS_ERR_INVALID_ARG
    assert status_of(lambda: A.abs_centroid_row_bytes(0, 0)) == A.ABS_ERR_INVALID_ARG
    h = Host()
    need_b = A.abs_workspace_bytes(h.kv, h.bmap, 64, A.ABS_OP_BUILD)
    need_s = A.abs_workspace_bytes(h.kv, h.bmap, 64, A.ABS_OP_SELECT)
    cap = A.abs_select_capacity(h.kv, h.bmap, 64)
    bad = [A.abs_centroids(codes=FAKE, scale=FAKE, lo=FAKE, format=5),
           A.abs_centroids(codes=FAKE, scale=FAKE, lo=FAKE, format=-1),
           A.abs_centroids(codes=FAKE, scale=FAKE, lo=FAKE, format=0, reserved0=1),
           A.abs_centroids(codes=FAKE + 8, scale=FAKE, lo=FAKE, format=2)]
    I = A.ABS_ERR_INVALID_ARG
    for c in bad:
        assert status_of(lambda: A.abs_build_centroids(h.kv, h.bmap, c, FAKE, need_b, 0)) == I
        assert status_of(lambda: A.abs_update_centroids(h.kv, h.bmap, c, 1, None, 0)) == I
        assert status_of(lambda: A.abs_score_select(h.kv, h.bmap, c, FAKE, 64, FAKE, cap, FAKE, FAKE, need_s,
                                                    0)) == I


def test_assign_block_sizes_follows_the_oracle_rule(oracle_mod):
    """The C host rule and the oracle's agree on random tables (fp32 recalls,
    a threshold exact in fp32) and on hand-made edge cases."""
    rng = np.random.default_rng(3)
    for _ in range(20):
        r = rng.uniform(0, 1, (3, 16)).astype(np.float32)
        r[1:] = np.minimum(1, r[0] * rng.uniform(0.8, 1.1, (2, 16))).astype(np.float32)
        r[:, 0] = 0.0
        np.testing.assert_array_equal(A.abs_assign_block_sizes(r, 0.9375),
                                      oracle_mod.assign_block_sizes(r.astype(np.float64), 0.9375))
    edge = np.array([[0.5, 0.5, 0.0], [0.46875, 0.25, 0.0], [0.25, 0.5, 0.0]], dtype=np.float32)
    np.testing.assert_array_equal(A.abs_assign_block_sizes(edge, 0.9375), [32, 64, 64])


def test_calibration_call_validation():
    I = A.ABS_ERR_INVALID_ARG
    ok = np.full((3, 4), 0.5, dtype=np.float32)
    assert status_of(lambda: A.abs_assign_block_sizes(ok, 0.0)) == I
    assert status_of(lambda: A.abs_assign_block_sizes(ok, float("nan"))) == I
    for bad in (1.5, -0.1, float("nan")):
        r = ok.copy()
        r[2, 1] = bad
        assert status_of(lambda: A.abs_assign_block_sizes(r, 0.95)) == I
    h = Host()
    assert status_of(lambda: A.abs_head_recall(h.kv, FAKE, None, FAKE, 0)) == I
    h.kv.num_q_heads = 3
    assert status_of(lambda: A.abs_head_recall(h.kv, FAKE, FAKE, FAKE, 0)) == I


def test_too_many_sequence_heads_is_unsupported():
    h = Host(seq_lens=(16,) * 8193, block_size=(16,) * 8, Hq=8)
    assert status_of(lambda: A.abs_total_blocks(h.kv, h.bmap)) == A.ABS_ERR_UNSUPPORTED
    h = Host(seq_lens=(16,) * 8192, block_size=(16,) * 8, Hq=8)
    assert A.abs_total_blocks(h.kv, h.bmap) == 8192 * 8


def test_too_many_blocks_per_head_is_unsupported():
    h = Host(seq_lens=(65537 * 16,), block_size=(16,), Hq=1, max_pages=65537)
    cap = A.abs_select_capacity(h.kv, h.bmap, 64)
    need = A.abs_workspace_bytes(h.kv, h.bmap, 64, A.ABS_OP_SELECT)
    assert status_of(lambda: A.abs_score_select(h.kv, h.bmap, h.cents, FAKE, 64, FAKE, cap, FAKE, FAKE, need,
                                                0)) == A.ABS_ERR_UNSUPPORTED


@pytest.mark.parametrize("cfg,splits,ppw,pipelined", [(1, 16, 8, 0), (2, 2, 64, 1), (3, 8, 32, 1), (4, 4, 32, 1)])
def test_launch_plan_of_the_workloads(cfg, splits, ppw, pipelined):
    """The launch shapes abs_select_decode takes for the 8B-shaped decode
    workloads (host sizing only: no GPU here, so the MI355X's 256 compute
    units are assumed): every one runs the top-K inside the decode launch."""
    from block_sparse_attention_abs_amd import workload as W
    w = W.PRESETS[cfg]
    bs = W.block_sizes_for(w, 0)
    h = Host(seq_lens=(w.context,) * w.batch, block_size=tuple(int(b) for b in bs), Hq=w.num_q_heads,
             D=w.head_dim, max_pages=w.context // 16)
    plan = A.abs_describe_launch(h.kv, h.bmap, w.token_budget)
    assert (plan["splits"], plan["pages_per_wg"], plan["pipelined"], plan["fused"]) == (splits, ppw, pipelined, 1)
    assert plan["chunk"] == 8 and plan["compute_units"] == 256
    assert plan["sel_cap"] == A.abs_select_capacity(h.kv, h.bmap, w.token_budget)
    assert plan["max_blocks"] == max(-(-w.context // int(b)) for b in bs)
    # every head reads budget / 16 pages, and the splits cover them
    assert splits * ppw >= w.token_budget // 16


def test_static_scratch_call_rejects_layers_beyond_its_size():
    """abs_select_decode_static checks the layer's scratch need against
    ABS_STATIC_SCRATCH_BYTES on the host, before touching any device."""
    import re as _re
    m = _re.search(r"#define ABS_STATIC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", open(HEADER).read())
    assert m and int(m.group(1)) << int(m.group(2)) == A.STATIC_SCRATCH_BYTES
    big = Host(seq_lens=(131072,) * 64, block_size=(16,) * 8, Hq=32, D=128, max_pages=8192)
    need = A.abs_workspace_bytes(big.kv, big.bmap, 4096, A.ABS_OP_SELECT_DECODE)
    assert need > A.STATIC_SCRATCH_BYTES
    cap = A.abs_select_capacity(big.kv, big.bmap, 4096)
    assert status_of(lambda: A.abs_select_decode_static(big.kv, big.bmap, big.cents, FAKE, 4096, 0.125, FAKE, cap,
                                                        FAKE, FAKE, None, 0)) == A.ABS_ERR_WORKSPACE
    assert "static scratch" in A.abs_last_error()
    h = Host()
    cap = A.abs_select_capacity(h.kv, h.bmap, 64)
    I = A.ABS_ERR_INVALID_ARG
    assert status_of(lambda: A.abs_select_decode_static(h.kv, h.bmap, h.cents, None, 64, 0.125, FAKE, cap, FAKE,
                                                        FAKE, None, 0)) == I
    assert status_of(lambda: A.abs_select_decode_static(h.kv, h.bmap, h.cents, FAKE, 64, 0.125, FAKE, cap - 1,
                                                        FAKE, FAKE, None, 0)) == I


def test_stage_calls_validation():
    """abs_estimate needs the centroid store and q; abs_topk_decode needs q,
    sel, sel_count, out, a large enough sel_cap and a finite sm_scale; both
    the select + decode workspace."""
    h = Host()
    need = A.abs_workspace_bytes(h.kv, h.bmap, 64, A.ABS_OP_SELECT_DECODE)
    cap = A.abs_select_capacity(h.kv, h.bmap, 64)
    I, W = A.ABS_ERR_INVALID_ARG, A.ABS_ERR_WORKSPACE
    assert status_of(lambda: A.abs_estimate(h.kv, h.bmap, None, FAKE, 64, FAKE, need, 0)) == I
    assert status_of(lambda: A.abs_estimate(h.kv, h.bmap, h.cents, None, 64, FAKE, need, 0)) == I
    assert status_of(lambda: A.abs_estimate(h.kv, h.bmap, h.cents, FAKE, 64, FAKE, need - 1, 0)) == W
    assert status_of(lambda: A.abs_estimate(h.kv, h.bmap, h.cents, FAKE, 0, FAKE, need, 0)) == I
    assert status_of(lambda: A.abs_topk_decode(h.kv, h.bmap, FAKE, 64, 0.125, FAKE, cap - 1, FAKE, FAKE, None, FAKE,
                                               need, 0)) == I
    assert status_of(lambda: A.abs_topk_decode(h.kv, h.bmap, FAKE, 64, 0.125, FAKE, cap, FAKE, None, None, FAKE,
                                               need, 0)) == I
    assert status_of(lambda: A.abs_topk_decode(h.kv, h.bmap, FAKE, 64, float("nan"), FAKE, cap, FAKE, FAKE, None,
                                               FAKE, need, 0)) == I
    assert status_of(lambda: A.abs_topk_decode(h.kv, h.bmap, FAKE, 64, 0.125, FAKE, cap, FAKE, FAKE, None, FAKE,
                                               need - 1, 0)) == W
    h.kv.v_cache = None
    assert status_of(lambda: A.abs_topk_decode(h.kv, h.bmap, FAKE, 64, 0.125, FAKE, cap, FAKE, FAKE, None, FAKE,
                                               need, 0)) == I


def test_reset_and_debug_switch_validation():
    h = Host()
    need_d = A.abs_workspace_bytes(h.kv, h.bmap, 64, A.ABS_OP_DECODE)
    need_sd = A.abs_workspace_bytes(h.kv, h.bmap, 64, A.ABS_OP_SELECT_DECODE)
    W, I = A.ABS_ERR_WORKSPACE, A.ABS_ERR_INVALID_ARG
    assert status_of(lambda: A.abs_reset_workspace(h.kv, h.bmap, 64, A.ABS_OP_DECODE, FAKE, need_d - 1, 0)) == W
    assert status_of(lambda: A.abs_reset_workspace(h.kv, h.bmap, 64, A.ABS_OP_SELECT_DECODE, FAKE, need_sd - 1,
                                                   0)) == W
    assert status_of(lambda: A.abs_reset_workspace(h.kv, h.bmap, 64, A.ABS_OP_SELECT_DECODE, None, need_sd, 0)) == W
    for op in (A.ABS_OP_BUILD, A.ABS_OP_SELECT, 9):
        assert status_of(lambda: A.abs_reset_workspace(h.kv, h.bmap, 64, op, FAKE, 1 << 30, 0)) == I
    assert status_of(lambda: A.abs_reset_workspace(h.kv, h.bmap, 0, A.ABS_OP_DECODE, FAKE, 1 << 30, 0)) == I
    assert A.abs_set_debug_checks(True) is False
    assert A.abs_set_debug_checks(False) is True
    assert A.abs_set_debug_checks(False) is False


def test_device_block_size_copy_is_optional():
    """The kernels take block sizes from the host copy; a NULL device copy is
    accepted (the validation that follows is the workspace size)."""
    h = Host()
    h.bmap.block_size = None
    need_b = A.abs_workspace_bytes(h.kv, h.bmap, 64, A.ABS_OP_BUILD)
    assert status_of(lambda: A.abs_build_centroids(h.kv, h.bmap, h.cents, FAKE, need_b - 1, 0)) == A.ABS_ERR_WORKSPACE


def test_status_strings():
    assert A.abs_status_str(A.ABS_OK) == "ok"
    assert A.abs_status_str(A.ABS_ERR_WORKSPACE) == "workspace too small"
    assert A.abs_status_str(99) == "unknown status"


def test_host_calls_from_plain_c(tmp_path):
    """tests/c/host_calls.c links libabs.so from C and calls every host-side
    function of abs.h; its results equal the binding's and the closed forms
    (N = ceil(L / bs), K = min(N, max(1, budget // bs)))."""
    exe = tmp_path / "host_calls"
    lib_dir = os.path.dirname(A.LIB_PATH)
    subprocess.run(["gcc", "-std=c11", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "c", "host_calls.c"), "-L", lib_dir, "-labs",
                    f"-Wl,-rpath,{lib_dir}", "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout
    got = {l.split()[0]: l.split()[1:] for l in out.splitlines()}
    lens, bs = [300, 77, 1], [16, 64]
    n = [-(-L // b) for L in lens for b in bs]
    assert int(got["total_blocks"][0]) == sum(n)
    assert [int(v) for v in got["offsets"]] == [0] + np.cumsum(n).tolist()
    ncap = [-(-512 // b) for _ in lens for b in bs]
    assert [int(v) for v in got["offsets_capacity"]] == [0] + np.cumsum(ncap).tolist()
    assert int(got["select_capacity"][0]) == max(min(-(-L // b), max(1, 100 // b)) for L in lens for b in bs)
    h = Host(seq_lens=lens, block_size=bs, Hq=8, D=128)
    assert [int(v) for v in got["workspace"]] == [A.abs_workspace_bytes(h.kv, h.bmap, 100, op) for op in range(3)]
    assert [int(v) for v in got["row_bytes"]] == [64, 64, 128, 64, 256]
    assert [int(v) for v in got["assign"]] == [32, 16, 64]
    plan = A.abs_describe_launch(h.kv, h.bmap, 100)
    assert [int(v) for v in got["plan"]] == [plan[k] for k in ("splits", "pages_per_wg", "chunk", "pipelined",
                                                               "fused", "score_workgroups", "max_blocks", "sel_cap")]
    assert got["debug_checks"] == ["0", "1"]
    assert int(got["status_page_size"][0]) == A.ABS_ERR_UNSUPPORTED
    assert int(got["status_block_size"][0]) == A.ABS_ERR_UNSUPPORTED
    assert int(got["status_capacity"][0]) == A.ABS_ERR_INVALID_ARG
    assert int(got["status_budget"][0]) == A.ABS_ERR_INVALID_ARG
    assert got["last_error_nonempty"] == ["1"]


def test_division_without_division_is_exact(tmp_path):
    """The kernels divide flat indices by Hkv and by the pages per workgroup
    with a multiply by a magic number (div_magic / fast_div, launch.hpp);
    tests/c/div_magic.cpp checks it against integer division for every
    divisor 1..64 and every dividend below 2^26, on the host."""
    import shutil
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not found")
    exe = tmp_path / "div_magic"
    subprocess.run([hipcc, "-O2", "-std=c++17", "--offload-arch=gfx950", "-I",
                    os.path.join(ROOT, "block_sparse_attention_abs_amd", "csrc"),
                    os.path.join(ROOT, "tests", "c", "div_magic.cpp"), "-o", str(exe)], check=True,
                   capture_output=True, timeout=600)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr


@pytest.mark.parametrize("args", [
    (0, 10, 4096, 4, 2, 1),          # null tile_addr
    (1, 10, 4096, 4, 2, 0),          # null xor_out
    (1, 10, 2048, 4, 2, 1),          # tile size other than 4096
    (1, 0, 4096, 4, 2, 1),           # no tiles
    (1, 10, 4096, 0, 2, 1),          # no workgroups
    (1, 10, 4096, 65536, 2, 1),      # too many workgroups
    (1, 10, 4096, 4, 3, 1),          # in_flight not 1, 2, 4 or 8
])
def test_gather_probe_rejects_bad_arguments(args):
    """abs_gather_tiles checks its arguments on the host before any launch
    (the pointers here are never dereferenced: each call fails first)."""
    addr, n, tile_bytes, wgs, in_flight, out = args
    st = status_of(lambda: A.abs_gather_tiles(addr, n, tile_bytes, wgs, in_flight, out, 0))
    assert st == A.ABS_ERR_INVALID_ARG
