"""Host logic of bench.py (no GPU): the one-GPU guard, the layer-copy count
that keeps the Infinity Cache cold, and the source list that keys the
measured traffic figure."""
import os
import re
import subprocess
import sys
from types import SimpleNamespace

import numpy as np

import bench

CSRC = os.path.join(bench.ROOT, "block_sparse_attention_abs_amd", "csrc")


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(bench.ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _layer(batch, context, dtype="bf16", kv_heads=8, head_dim=128, pages=None):
    sz = 2 if dtype == "bf16" else 4
    pages = pages if pages is not None else batch * context // 16
    nbytes = pages * kv_heads * 16 * head_dim * sz
    x = SimpleNamespace(dtype=dtype, seq_lens=np.full(batch, context), k_cache=SimpleNamespace(nbytes=nbytes),
                        v_cache=SimpleNamespace(nbytes=nbytes))
    return x


def test_layer_copies_cover_twice_the_infinity_cache():
    # 128K x 4, budget 4096: 4 * 8 * 4096 tokens of K and V = 64 MiB per step,
    # so 8 copies (the minimum) already pass 2 x 256 MiB
    w = SimpleNamespace(token_budget=4096, num_kv_heads=8, head_dim=128)
    assert bench.auto_replicas(w, _layer(4, 131072)) == 8
    # 32K x 1, budget 2048: 8 MiB per step, 64 copies
    w = SimpleNamespace(token_budget=2048, num_kv_heads=8, head_dim=128)
    assert bench.auto_replicas(w, _layer(1, 32768)) == 64
    # capped so the copies hold at most 64 GiB of K/V
    x = _layer(1, 32768, pages=1 << 15)                      # 1 GiB per cache, 2 GiB per copy
    assert bench.auto_replicas(w, x) == 32


def _local_includes(name, seen):
    seen.add(name)
    with open(os.path.join(CSRC, name)) as f:
        for inc in re.findall(r'^#include "([^"]+)"', f.read(), flags=re.M):
            if inc not in seen and os.path.exists(os.path.join(CSRC, inc)):
                _local_includes(inc, seen)
    return seen


def test_traffic_key_covers_every_decode_source():
    # the measured traffic figure is reported only while these sources are
    # unchanged: every header the decode kernels include must be among them
    srcs = _local_includes("decode.hip", set())
    assert srcs <= set(bench.KERNEL_SOURCES), srcs - set(bench.KERNEL_SOURCES)
    h = bench.kernel_source_hash()
    assert re.fullmatch(r"[0-9a-f]{16}", h)


def test_traffic_figures_name_the_shape_they_were_measured_on():
    # a figure is looked up by (workload, batch, context, block map, source
    # hash): a run at another batch or context must not find it
    from block_sparse_attention_abs_amd.workload import PRESETS
    names = {w.name for w in PRESETS}
    for key, nbytes in bench.TRAFFIC.items():
        name, batch, context, block_map, h = key
        assert name in names and isinstance(batch, int) and batch > 0 and isinstance(context, int)
        assert block_map in ("drawn", "16", "32", "64") and re.fullmatch(r"[0-9a-f]{16}", h)
        assert nbytes > 0


def _counter_csv(path, rows):
    import csv
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for r in rows:
            w.writerow(r)


def test_traffic_summary_scales_by_the_copy_and_counts_requests(tmp_path, capsys):
    # counter files of a made-up command: a copy of 1 MiB (three dispatches)
    # and two dispatches of a kernel; FETCH_SIZE reads half a copy's bytes
    from block_sparse_attention_abs_amd import traffic
    copy, kern = "__amd_rocclr_copyBuffer", "void absk::k_demo<4>(int)"
    mib = 1 << 20
    _counter_csv(tmp_path / "f.csv", [(1, copy, "FETCH_SIZE", 512), (2, copy, "FETCH_SIZE", 512),
                                      (3, copy, "FETCH_SIZE", 512), (4, kern, "FETCH_SIZE", 100),
                                      (5, kern, "FETCH_SIZE", 300)])
    _counter_csv(tmp_path / "w.csv", [(1, copy, "WRITE_SIZE", 1024), (2, copy, "WRITE_SIZE", 1024),
                                      (3, copy, "WRITE_SIZE", 1024), (4, kern, "WRITE_SIZE", 10),
                                      (5, kern, "WRITE_SIZE", 30)])
    req = []
    for d in (1, 2, 3):
        req += [(d, copy, "TCC_EA0_RDREQ_32B", 0), (d, copy, "TCC_EA0_RDREQ_64B", 0),
                (d, copy, "TCC_EA0_RDREQ_128B", mib // 128), (d, copy, "TCC_EA0_RDREQ", mib // 128)]
    # the kernel's two dispatches: 10 x 32 B + 20 x 64 B + 1000 x 128 B, and 3x that
    for d, k in ((4, 1), (5, 3)):
        req += [(d, kern, "TCC_EA0_RDREQ_32B", 10 * k), (d, kern, "TCC_EA0_RDREQ_64B", 20 * k),
                (d, kern, "TCC_EA0_RDREQ_128B", 1000 * k), (d, kern, "TCC_EA0_RDREQ", 1030 * k)]
    _counter_csv(tmp_path / "r.csv", req)
    import sys as _sys
    argv = _sys.argv
    _sys.argv = ["traffic", "bytes", str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), "--copy-bytes", str(mib),
                 "--rdreq", str(tmp_path / "r.csv")]
    try:
        traffic.main()
    finally:
        _sys.argv = argv
    out = capsys.readouterr().out
    assert "scale 2.0000 (read), 1.0000 (write)" in out
    assert f"by read requests (32/64/128 B): {mib} B (1.0000" in out
    row = [l for l in out.splitlines() if l.startswith("| k_demo<4>")][0].split("|")
    cells = [c.strip() for c in row[1:-1]]
    # mean FETCH 200 KiB x 2 = 409600 B read; mean WRITE 20 KiB = 20480 B written
    assert cells[1] == "2" and cells[4] == "409600" and cells[5] == "20480" and cells[6] == "430080"
    # request bytes: mean over the two dispatches of (320 + 1280 + 128000) x k, k = 1 and 3
    assert cells[7] == str(2 * (320 + 1280 + 128000))


def test_selected_tiles_follow_the_page_table():
    """The gather reference's tile list: for each selected block, the pages
    its tokens cover (the last one cut at L), each page's K tile then V tile
    at ((page id x Hkv + head) x tile bytes) from the cache bases."""
    page_table = np.array([[5, 2, 7, -1]], dtype=np.int32)
    seq_lens = np.array([40], dtype=np.int32)                  # 3 pages, the last holding 8 tokens
    block_size = np.array([16, 32], dtype=np.int32)            # two KV heads
    sel = np.array([[[1, 2], [0, -1]]], dtype=np.int32)
    cnt = np.array([[2, 1]], dtype=np.int32)
    a, o, is_k = bench.selected_tiles(page_table, seq_lens, block_size, 4096, sel, cnt, 1_000_000, 2_000_000)
    # head 0 (16-token blocks): block 1 -> page 1 (id 2), block 2 -> tokens 32..39 -> page 2 (id 7);
    # head 1 (32-token blocks): block 0 -> pages 0, 1 (ids 5, 2)
    want_o = [(2 * 2 + 0) * 4096, (7 * 2 + 0) * 4096, (5 * 2 + 1) * 4096, (2 * 2 + 1) * 4096]
    assert o.tolist() == [x for v in want_o for x in (v, v)]
    assert is_k.tolist() == [True, False] * 4
    assert a.tolist() == [(1_000_000 if k else 2_000_000) + v for v, k in zip(o.tolist(), is_k.tolist())]
