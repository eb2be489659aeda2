"""CPU oracle for the AB-Sparse decode path (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg use this
package.  It wraps ``abs_oracle.c`` (plain C, fp64, no code shared with the
HIP library) through ctypes on numpy host arrays.  Every function mirrors one
stage of Figure 1 of the AB-Sparse page: centroid, quantization, score,
top-K selection, sparse attention; the readings it takes are listed in the C
source next to each stage.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "abs_oracle.c")
_LIB_PATH = os.environ.get("ABS_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
GCC_CMD = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-o", _LIB_PATH, _SRC, "-lm"]

_lib = None


def build(force: bool = False) -> str:
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        subprocess.run(GCC_CMD, check=True)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        build()
        L = C.CDLL(_LIB_PATH)
        P = C.c_void_p
        i32, i64 = C.c_int, C.c_int64
        L.oracle_total_blocks.restype = i64
        L.oracle_total_blocks.argtypes = [i32, i32, P, P]
        L.oracle_k.restype = i64
        L.oracle_k.argtypes = [i64, i32, i32]
        L.oracle_centroids.argtypes = [i32, i32, i32, i32, i32, P, P, P, P, P]
        L.oracle_quantize.argtypes = [i32, i32, i32, P, P, P, P, P, P]
        L.oracle_update.argtypes = [i32, i32, i32, i32, i32, i32, P, P, P, P, P, P, P, P, P, P]
        L.oracle_quantize_fmt.argtypes = [i32, i32, i32, i32, P, P, P, P, P, P, P]
        L.oracle_scores_dense.argtypes = [i32, i32, i32, i32, i32, P, P, P, P, P]
        L.oracle_attention_mass.argtypes = [i32, i32, i32, i32, i32, i32, P, P, P, P, P, P, i32, P, C.c_double, P]
        L.oracle_scores.argtypes = [i32, i32, i32, i32, i32, P, P, P, P, P, P, P]
        L.oracle_select.argtypes = [i32, i32, P, P, i32, P, P, i32, P]
        L.oracle_attend.argtypes = [i32, i32, i32, i32, i32, i32, P, P, P, P, P, P, P, i32, P,
                                    C.c_double, P, P]
        L.oracle_max_threads.restype = i32
        L.oracle_set_threads.argtypes = [i32]
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags.c_contiguous
    return a.ctypes.data_as(C.c_void_p)


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.int32)


def _is_bf16(dtype: str) -> int:
    assert dtype in ("f32", "bf16")
    return 1 if dtype == "bf16" else 0


def _store(a: np.ndarray, dtype: str) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.uint16 if dtype == "bf16" else np.float32)


def set_threads(n: int) -> None:
    lib().oracle_set_threads(int(n))


def max_threads() -> int:
    return int(lib().oracle_max_threads())


def total_blocks(seq_lens, block_size) -> int:
    sl, bs = _i32(seq_lens), _i32(block_size)
    return int(lib().oracle_total_blocks(len(sl), len(bs), _p(sl), _p(bs)))


def k_of(L: int, bs: int, budget: int) -> int:
    return int(lib().oracle_k(int(L), int(bs), int(budget)))


def block_rows(seq_lens, block_size):
    """[(b, h, first_row, N)] in the CSR order the oracle stores blocks in."""
    rows, r = [], 0
    for b, L in enumerate(seq_lens):
        for h, bs in enumerate(block_size):
            n = (int(L) + int(bs) - 1) // int(bs)
            rows.append((b, h, r, n))
            r += n
    return rows


def centroids(k_cache, page_table, seq_lens, block_size, dtype: str) -> np.ndarray:
    """fp32 centroids [total_blocks][D]."""
    k = _store(k_cache, dtype)
    pt, sl, bs = _i32(page_table), _i32(seq_lens), _i32(block_size)
    B, Hkv, D = pt.shape[0], k.shape[1], k.shape[3]
    out = np.empty((total_blocks(sl, bs), D), dtype=np.float32)
    lib().oracle_centroids(B, Hkv, D, pt.shape[1], _is_bf16(dtype), _p(k), _p(pt), _p(sl), _p(bs), _p(out))
    return out


@dataclass
class Quantized:
    codes: np.ndarray   # uint8 [total_blocks][D], values 0..15
    scale: np.ndarray   # f32 [B][Hkv][D]
    lo: np.ndarray      # f32 [B][Hkv][D]


def quantize(cents: np.ndarray, seq_lens, block_size) -> Quantized:
    c = np.ascontiguousarray(cents, dtype=np.float32)
    sl, bs = _i32(seq_lens), _i32(block_size)
    B, Hkv, D = len(sl), len(bs), c.shape[1]
    codes = np.empty(c.shape, dtype=np.uint8)
    scale = np.empty((B, Hkv, D), dtype=np.float32)
    lo = np.empty((B, Hkv, D), dtype=np.float32)
    lib().oracle_quantize(B, Hkv, D, _p(sl), _p(bs), _p(c), _p(codes), _p(scale), _p(lo))
    return Quantized(codes, scale, lo)


def csr_offsets(seq_lens, block_size, capacity_tokens=None) -> np.ndarray:
    """Row offsets [B*Hkv + 1] of each (b, h)'s blocks, b-major; with
    capacity_tokens, each head gets room for ceil(capacity / bs) rows."""
    out, r = [], 0
    for L in seq_lens:
        for bs in block_size:
            out.append(r)
            n = int(capacity_tokens) if capacity_tokens is not None else int(L)
            r += (n + int(bs) - 1) // int(bs)
    out.append(r)
    return np.asarray(out, dtype=np.int64)


FORMATS = {"int4": 0, "int4_sym": 1, "int8": 2, "int4_tensor": 3, "bf16": 4}


def update(k_cache, page_table, seq_lens, prev_lens, block_size, row_off, quant, dtype: str, fmt: str = "int4"):
    """Centroids kept current after appends (see oracle_update): returns a copy
    of quant.codes ([rows][D] code values in format fmt, rows addressed through
    row_off) with the blocks holding tokens [prev_b - 1, L_b) recomputed, and
    out_of_range [B][Hkv]."""
    k = _store(k_cache, dtype)
    pt, sl, pl, bs = _i32(page_table), _i32(seq_lens), _i32(prev_lens), _i32(block_size)
    off = np.ascontiguousarray(row_off, dtype=np.int64)
    B, Hkv, D = pt.shape[0], k.shape[1], k.shape[3]
    codes = np.array(quant.codes, dtype=np.uint16, copy=True, order="C")
    assert codes.shape[0] >= off[-1] and codes.shape[1] == D
    assert ((pl >= 1) & (pl <= sl)).all()
    sc = np.ascontiguousarray(quant.scale, dtype=np.float32)
    lo = np.ascontiguousarray(quant.lo, dtype=np.float32)
    oor = np.zeros((B, Hkv), dtype=np.int32)
    lib().oracle_update(FORMATS[fmt], B, Hkv, D, pt.shape[1], _is_bf16(dtype), _p(k), _p(pt), _p(sl), _p(pl),
                        _p(bs), _p(off), _p(sc), _p(lo), _p(codes), _p(oor))
    return codes.astype(np.asarray(quant.codes).dtype), oor




@dataclass
class QuantizedFmt:
    fmt: str
    codes: np.ndarray   # uint16 [total_blocks][D]: code values (int4_sym: q + 8), bf16 bit patterns
    scale: np.ndarray   # f32 [B][Hkv][D] (bf16: 0)
    lo: np.ndarray      # f32 [B][Hkv][D] (int4_sym: -8*scale; bf16: 0)
    deq: np.ndarray     # fp64 [total_blocks][D] dequantized centroids


def quantize_fmt(cents: np.ndarray, seq_lens, block_size, fmt: str) -> QuantizedFmt:
    """Centroids in one of the formats of oracle_quantize_fmt."""
    c = np.ascontiguousarray(cents, dtype=np.float32)
    sl, bs = _i32(seq_lens), _i32(block_size)
    B, Hkv, D = len(sl), len(bs), c.shape[1]
    codes = np.empty(c.shape, dtype=np.uint16)
    scale = np.empty((B, Hkv, D), dtype=np.float32)
    lo = np.empty((B, Hkv, D), dtype=np.float32)
    deq = np.empty(c.shape, dtype=np.float64)
    lib().oracle_quantize_fmt(FORMATS[fmt], B, Hkv, D, _p(sl), _p(bs), _p(c), _p(codes), _p(scale), _p(lo),
                              _p(deq))
    return QuantizedFmt(fmt, codes, scale, lo, deq)


def scores_dense(q, deq: np.ndarray, seq_lens, block_size, dtype: str) -> np.ndarray:
    """fp64 scores from dequantized centroids of any format."""
    qq = _store(q, dtype)
    sl, bs = _i32(seq_lens), _i32(block_size)
    B, Hq, D = qq.shape
    dq = np.ascontiguousarray(deq, dtype=np.float64)
    out = np.empty(dq.shape[0], dtype=np.float64)
    lib().oracle_scores_dense(B, Hq, len(bs), D, _is_bf16(dtype), _p(qq), _p(sl), _p(bs), _p(dq), _p(out))
    return out


def scores(q, quant: Quantized, seq_lens, block_size, dtype: str) -> np.ndarray:
    """fp64 importance scores [total_blocks]."""
    qq = _store(q, dtype)
    sl, bs = _i32(seq_lens), _i32(block_size)
    B, Hq, D = qq.shape
    codes = np.ascontiguousarray(quant.codes, dtype=np.uint8)
    sc = np.ascontiguousarray(quant.scale, dtype=np.float32)
    lo = np.ascontiguousarray(quant.lo, dtype=np.float32)
    out = np.empty(codes.shape[0], dtype=np.float64)
    lib().oracle_scores(B, Hq, len(bs), D, _is_bf16(dtype), _p(qq), _p(sl), _p(bs), _p(codes), _p(sc),
                        _p(lo), _p(out))
    return out


def select(sc: np.ndarray, seq_lens, block_size, budget: int, sel_cap: int):
    """Top-K per (b, h): (sel int32 [B][Hkv][sel_cap] ascending, -1 padded; count int32 [B][Hkv])."""
    s = np.ascontiguousarray(sc, dtype=np.float64)
    sl, bs = _i32(seq_lens), _i32(block_size)
    B, Hkv = len(sl), len(bs)
    sel = np.full((B, Hkv, sel_cap), -1, dtype=np.int32)
    cnt = np.zeros((B, Hkv), dtype=np.int32)
    lib().oracle_select(B, Hkv, _p(sl), _p(bs), int(budget), _p(s), _p(sel), int(sel_cap), _p(cnt))
    return sel, cnt


def attend(q, k_cache, v_cache, page_table, seq_lens, block_size, sel, count, sm_scale: float,
           dtype: str):
    """Sparse attention over the selected blocks: (out fp64 [B][Hq][D], lse fp64 [B][Hq])."""
    qq, k, v = _store(q, dtype), _store(k_cache, dtype), _store(v_cache, dtype)
    pt, sl, bs = _i32(page_table), _i32(seq_lens), _i32(block_size)
    se, cn = _i32(sel), _i32(count)
    B, Hq, D = qq.shape
    out = np.empty((B, Hq, D), dtype=np.float64)
    lse = np.empty((B, Hq), dtype=np.float64)
    lib().oracle_attend(B, Hq, k.shape[1], D, pt.shape[1], _is_bf16(dtype), _p(qq), _p(k), _p(v), _p(pt),
                        _p(sl), _p(bs), _p(se), se.shape[-1], _p(cn), float(sm_scale), _p(out), _p(lse))
    return out, lse


def attention_mass(q, k_cache, page_table, seq_lens, block_size, sel, count, sm_scale: float,
                   dtype: str) -> np.ndarray:
    """Share of each query head's exact attention over all its tokens that
    the selection keeps (see oracle_attention_mass): fp64 [B][Hq]."""
    qq, k = _store(q, dtype), _store(k_cache, dtype)
    pt, sl, bs = _i32(page_table), _i32(seq_lens), _i32(block_size)
    se, cn = _i32(sel), _i32(count)
    B, Hq, D = qq.shape
    mass = np.empty((B, Hq), dtype=np.float64)
    lib().oracle_attention_mass(B, Hq, k.shape[1], D, pt.shape[1], _is_bf16(dtype), _p(qq), _p(k), _p(pt), _p(sl),
                                _p(bs), _p(se), se.shape[-1], _p(cn), float(sm_scale), _p(mass))
    return mass


CALIBRATION_SIZES = (16, 32, 64)


def head_recall(x, block_size: int, budget: int, sm_scale: float, fmt: str = "int4") -> np.ndarray:
    """Recall of every KV head when all heads use `block_size` (Figure 3's
    x axis): run centroids, quantization (format fmt), estimation and top-K
    at that block size, then average the attention mass kept over the
    sequences and the head's query group.  fp64 [Hkv]."""
    Hkv = x.k_cache.shape[1]
    bs = np.full(Hkv, int(block_size), dtype=np.int32)
    c = centroids(x.k_cache, x.page_table, x.seq_lens, bs, x.dtype)
    qf = quantize_fmt(c, x.seq_lens, bs, fmt)
    s = scores_dense(x.q, qf.deq, x.seq_lens, bs, x.dtype)
    cap = sel_capacity(x.seq_lens, bs, budget)
    sel, cnt = select(s, x.seq_lens, bs, budget, cap)
    mass = attention_mass(x.q, x.k_cache, x.page_table, x.seq_lens, bs, sel, cnt, sm_scale, x.dtype)
    B, Hq = mass.shape
    G = Hq // Hkv
    return mass.reshape(B, Hkv, G).mean(axis=(0, 2))


def assign_block_sizes(recall: np.ndarray, threshold: float) -> np.ndarray:
    """The allocation rule (reading of Figure 3 and the heatmap after it):
    recall[k][h] is head h's recall at block size CALIBRATION_SIZES[k]; its
    normalized recall is recall / recall at 16 (1 when that is 0); the head
    gets the largest block size whose normalized recall is >= threshold,
    else 16.  int32 [Hkv]."""
    r = np.asarray(recall, dtype=np.float64)
    out = np.full(r.shape[1], CALIBRATION_SIZES[0], dtype=np.int32)
    for h in range(r.shape[1]):
        base = r[0, h]
        for k in range(len(CALIBRATION_SIZES) - 1, 0, -1):
            norm = r[k, h] / base if base > 0 else 1.0
            if norm >= threshold:
                out[h] = CALIBRATION_SIZES[k]
                break
    return out


def sel_capacity(seq_lens, block_size, budget: int) -> int:
    return max(k_of(L, bs, budget) for L in seq_lens for bs in block_size)


@dataclass
class Pipeline:
    cents: np.ndarray
    quant: Quantized
    scores: np.ndarray
    sel: np.ndarray
    count: np.ndarray
    out: np.ndarray
    lse: np.ndarray


def run(x, sm_scale: float | None = None, budget: int | None = None) -> Pipeline:
    """The whole decode path on one layer's inputs (a workload.LayerInputs)."""
    D = x.q.shape[-1]
    sm = float(np.float32(1.0 / np.sqrt(D))) if sm_scale is None else float(sm_scale)
    bud = x.workload.token_budget if budget is None else int(budget)
    c = centroids(x.k_cache, x.page_table, x.seq_lens, x.block_size, x.dtype)
    qz = quantize(c, x.seq_lens, x.block_size)
    s = scores(x.q, qz, x.seq_lens, x.block_size, x.dtype)
    cap = sel_capacity(x.seq_lens, x.block_size, bud)
    sel, cnt = select(s, x.seq_lens, x.block_size, bud, cap)
    out, lse = attend(x.q, x.k_cache, x.v_cache, x.page_table, x.seq_lens, x.block_size, sel, cnt, sm, x.dtype)
    return Pipeline(c, qz, s, sel, cnt, out, lse)
