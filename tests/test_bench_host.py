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
