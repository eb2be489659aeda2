"""Python binding of libabs.so, the AB-Sparse decode library (include/abs.h).

Argument marshalling only: the functions below have the C names, take the
same descriptors (as ctypes structures) and raw device pointers, and call
straight into the library.  Every step of the decode path runs in the HIP
kernels behind those calls; there is no fallback.  If libabs.so is missing
or does not load, every call raises.

`PagedKV` is a convenience holder that keeps torch tensors alive and fills
the descriptors from them (PyTorch supplies device memory and streams only).
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libabs.so")

ABS_OK, ABS_ERR_INVALID_ARG, ABS_ERR_UNSUPPORTED, ABS_ERR_WORKSPACE, ABS_ERR_HIP = range(5)
ABS_F32, ABS_BF16 = 0, 1
ABS_OP_BUILD, ABS_OP_SELECT, ABS_OP_DECODE, ABS_OP_SELECT_DECODE = 0, 1, 2, 3
# abs_centroid_format, by name
CENTROID_FORMATS = {"int4": 0, "int4_sym": 1, "int8": 2, "int4_tensor": 3, "bf16": 4}

EXPORTS = ("abs_status_str", "abs_last_error", "abs_total_blocks", "abs_centroid_offsets",
           "abs_centroid_offsets_capacity", "abs_centroid_row_bytes", "abs_select_capacity", "abs_workspace_bytes", "abs_build_centroids",
           "abs_update_centroids", "abs_score_select", "abs_sparse_decode", "abs_select_decode",
           "abs_estimate", "abs_topk_decode", "abs_select_decode_static", "abs_describe_launch", "abs_reset_workspace", "abs_set_debug_checks",
           "abs_head_recall", "abs_assign_block_sizes", "abs_gather_tiles")


class abs_paged_kv(C.Structure):
    _fields_ = [("num_seqs", C.c_int32), ("num_q_heads", C.c_int32), ("num_kv_heads", C.c_int32),
                ("head_dim", C.c_int32), ("page_size", C.c_int32), ("max_pages_per_seq", C.c_int32),
                ("num_pages", C.c_int64), ("kv_dtype", C.c_int32), ("reserved0", C.c_int32),
                ("k_cache", C.c_void_p), ("v_cache", C.c_void_p), ("page_table", C.c_void_p),
                ("seq_lens", C.c_void_p), ("seq_lens_host", C.c_void_p)]


class abs_block_map(C.Structure):
    _fields_ = [("block_size_host", C.c_void_p), ("block_size", C.c_void_p), ("centroid_off", C.c_void_p)]


class abs_centroids(C.Structure):
    _fields_ = [("codes", C.c_void_p), ("scale", C.c_void_p), ("lo", C.c_void_p), ("format", C.c_int32),
                ("reserved0", C.c_int32)]


class abs_launch_plan(C.Structure):
    _fields_ = [("splits", C.c_int32), ("pages_per_wg", C.c_int32), ("chunk", C.c_int32),
                ("pipelined", C.c_int32), ("fused", C.c_int32), ("score_workgroups", C.c_int32),
                ("max_blocks", C.c_int32), ("sel_cap", C.c_int32), ("compute_units", C.c_int32),
                ("reserved", C.c_int32 * 7)]


class AbsError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: status {status} ({detail})")
        self.status = status


_lib = None


def lib():
    """Load libabs.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m block_sparse_attention_abs_amd.build`")
        L = C.CDLL(LIB_PATH)
        P, KV, MAP, CEN = C.c_void_p, C.POINTER(abs_paged_kv), C.POINTER(abs_block_map), C.POINTER(abs_centroids)
        i32, st = C.c_int32, C.c_int
        L.abs_status_str.restype = C.c_char_p
        L.abs_status_str.argtypes = [st]
        L.abs_last_error.restype = C.c_char_p
        L.abs_last_error.argtypes = []
        L.abs_total_blocks.restype = st
        L.abs_total_blocks.argtypes = [KV, MAP, C.POINTER(C.c_int64)]
        L.abs_centroid_offsets.restype = st
        L.abs_centroid_offsets.argtypes = [KV, MAP, P]
        L.abs_centroid_offsets_capacity.restype = st
        L.abs_centroid_offsets_capacity.argtypes = [KV, MAP, i32, P]
        L.abs_centroid_row_bytes.restype = st
        L.abs_centroid_row_bytes.argtypes = [i32, i32, C.POINTER(C.c_int64)]
        L.abs_select_capacity.restype = st
        L.abs_select_capacity.argtypes = [KV, MAP, i32, C.POINTER(C.c_int32)]
        L.abs_workspace_bytes.restype = st
        L.abs_workspace_bytes.argtypes = [KV, MAP, i32, st, C.POINTER(C.c_size_t)]
        L.abs_build_centroids.restype = st
        L.abs_build_centroids.argtypes = [KV, MAP, CEN, P, C.c_size_t, P]
        L.abs_update_centroids.restype = st
        L.abs_update_centroids.argtypes = [KV, MAP, CEN, i32, P, P]
        L.abs_score_select.restype = st
        L.abs_score_select.argtypes = [KV, MAP, CEN, P, i32, P, i32, P, P, C.c_size_t, P]
        L.abs_sparse_decode.restype = st
        L.abs_sparse_decode.argtypes = [KV, MAP, P, P, i32, P, i32, C.c_float, P, P, P, C.c_size_t, P]
        L.abs_select_decode.restype = st
        L.abs_select_decode.argtypes = [KV, MAP, CEN, P, i32, C.c_float, P, i32, P, P, P, P, C.c_size_t, P]
        L.abs_estimate.restype = st
        L.abs_estimate.argtypes = [KV, MAP, CEN, P, i32, P, C.c_size_t, P]
        L.abs_topk_decode.restype = st
        L.abs_topk_decode.argtypes = [KV, MAP, P, i32, C.c_float, P, i32, P, P, P, P, C.c_size_t, P]
        L.abs_select_decode_static.restype = st
        L.abs_select_decode_static.argtypes = [KV, MAP, CEN, P, i32, C.c_float, P, i32, P, P, P, P]
        L.abs_describe_launch.restype = st
        L.abs_describe_launch.argtypes = [KV, MAP, i32, C.POINTER(abs_launch_plan)]
        L.abs_reset_workspace.restype = st
        L.abs_reset_workspace.argtypes = [KV, MAP, i32, st, P, C.c_size_t, P]
        L.abs_set_debug_checks.restype = i32
        L.abs_set_debug_checks.argtypes = [i32]
        L.abs_head_recall.restype = st
        L.abs_head_recall.argtypes = [KV, P, P, P, P]
        L.abs_assign_block_sizes.restype = st
        L.abs_assign_block_sizes.argtypes = [i32, P, C.c_float, P]
        L.abs_gather_tiles.restype = st
        L.abs_gather_tiles.argtypes = [P, i32, i32, i32, i32, P, P]
        _lib = L
    return _lib


def _check(status: int, where: str) -> None:
    if status != ABS_OK:
        L = lib()
        raise AbsError(status, where, f"{L.abs_status_str(status).decode()}: {L.abs_last_error().decode()}")


# ---- the C calls, same names ------------------------------------------------

def abs_status_str(status: int) -> str:
    return lib().abs_status_str(status).decode()


def abs_last_error() -> str:
    return lib().abs_last_error().decode()


def abs_total_blocks(kv: abs_paged_kv, bmap: abs_block_map) -> int:
    n = C.c_int64()
    _check(lib().abs_total_blocks(C.byref(kv), C.byref(bmap), C.byref(n)), "abs_total_blocks")
    return n.value


def abs_centroid_offsets(kv: abs_paged_kv, bmap: abs_block_map) -> np.ndarray:
    off = np.zeros(kv.num_seqs * kv.num_kv_heads + 1, dtype=np.int64)
    _check(lib().abs_centroid_offsets(C.byref(kv), C.byref(bmap), off.ctypes.data), "abs_centroid_offsets")
    return off


def abs_centroid_offsets_capacity(kv: abs_paged_kv, bmap: abs_block_map, capacity_tokens: int) -> np.ndarray:
    off = np.zeros(kv.num_seqs * kv.num_kv_heads + 1, dtype=np.int64)
    _check(lib().abs_centroid_offsets_capacity(C.byref(kv), C.byref(bmap), capacity_tokens, off.ctypes.data),
           "abs_centroid_offsets_capacity")
    return off


def abs_centroid_row_bytes(head_dim: int, fmt: int) -> int:
    n = C.c_int64()
    _check(lib().abs_centroid_row_bytes(head_dim, fmt, C.byref(n)), "abs_centroid_row_bytes")
    return n.value


def abs_select_capacity(kv: abs_paged_kv, bmap: abs_block_map, token_budget: int) -> int:
    cap = C.c_int32()
    _check(lib().abs_select_capacity(C.byref(kv), C.byref(bmap), token_budget, C.byref(cap)),
           "abs_select_capacity")
    return cap.value


def abs_workspace_bytes(kv: abs_paged_kv, bmap: abs_block_map, token_budget: int, op: int) -> int:
    n = C.c_size_t()
    _check(lib().abs_workspace_bytes(C.byref(kv), C.byref(bmap), token_budget, op, C.byref(n)),
           "abs_workspace_bytes")
    return n.value


def abs_build_centroids(kv, bmap, cents, ws_ptr: int, ws_bytes: int, stream: int) -> None:
    _check(lib().abs_build_centroids(C.byref(kv), C.byref(bmap), C.byref(cents), ws_ptr, ws_bytes, stream),
           "abs_build_centroids")


def abs_update_centroids(kv, bmap, cents, appended: int, out_of_range_ptr: Optional[int], stream: int) -> None:
    _check(lib().abs_update_centroids(C.byref(kv), C.byref(bmap), C.byref(cents), appended, out_of_range_ptr,
                                      stream), "abs_update_centroids")


def abs_score_select(kv, bmap, cents, q_ptr: int, token_budget: int, sel_ptr: int, sel_cap: int,
                     count_ptr: int, ws_ptr: int, ws_bytes: int, stream: int) -> None:
    _check(lib().abs_score_select(C.byref(kv), C.byref(bmap), C.byref(cents), q_ptr, token_budget, sel_ptr,
                                  sel_cap, count_ptr, ws_ptr, ws_bytes, stream), "abs_score_select")


def abs_sparse_decode(kv, bmap, q_ptr: int, sel_ptr: int, sel_cap: int, count_ptr: int, token_budget: int,
                      sm_scale: float, out_ptr: int, lse_ptr: Optional[int], ws_ptr: int, ws_bytes: int,
                      stream: int) -> None:
    _check(lib().abs_sparse_decode(C.byref(kv), C.byref(bmap), q_ptr, sel_ptr, sel_cap, count_ptr, token_budget,
                                   sm_scale, out_ptr, lse_ptr, ws_ptr, ws_bytes, stream), "abs_sparse_decode")


def abs_select_decode(kv, bmap, cents, q_ptr: int, token_budget: int, sm_scale: float, sel_ptr: int, sel_cap: int,
                      count_ptr: int, out_ptr: int, lse_ptr: Optional[int], ws_ptr: int, ws_bytes: int,
                      stream: int) -> None:
    _check(lib().abs_select_decode(C.byref(kv), C.byref(bmap), C.byref(cents), q_ptr, token_budget, sm_scale,
                                   sel_ptr, sel_cap, count_ptr, out_ptr, lse_ptr, ws_ptr, ws_bytes, stream),
           "abs_select_decode")


def abs_estimate(kv, bmap, cents, q_ptr: int, token_budget: int, ws_ptr: int, ws_bytes: int, stream: int) -> None:
    _check(lib().abs_estimate(C.byref(kv), C.byref(bmap), C.byref(cents) if cents is not None else None, q_ptr,
                              token_budget, ws_ptr, ws_bytes, stream), "abs_estimate")


def abs_topk_decode(kv, bmap, q_ptr: int, token_budget: int, sm_scale: float, sel_ptr: int, sel_cap: int,
                    count_ptr: int, out_ptr: int, lse_ptr: Optional[int], ws_ptr: int, ws_bytes: int,
                    stream: int) -> None:
    _check(lib().abs_topk_decode(C.byref(kv), C.byref(bmap), q_ptr, token_budget, sm_scale, sel_ptr, sel_cap,
                                 count_ptr, out_ptr, lse_ptr, ws_ptr, ws_bytes, stream), "abs_topk_decode")


STATIC_SCRATCH_BYTES = 16 << 20   # ABS_STATIC_SCRATCH_BYTES


def abs_select_decode_static(kv, bmap, cents, q_ptr: int, token_budget: int, sm_scale: float, sel_ptr: int,
                             sel_cap: int, count_ptr: int, out_ptr: int, lse_ptr: Optional[int], stream: int) -> None:
    _check(lib().abs_select_decode_static(C.byref(kv), C.byref(bmap), C.byref(cents), q_ptr, token_budget, sm_scale,
                                          sel_ptr, sel_cap, count_ptr, out_ptr, lse_ptr, stream),
           "abs_select_decode_static")


def abs_describe_launch(kv, bmap, token_budget: int) -> dict:
    plan = abs_launch_plan()
    _check(lib().abs_describe_launch(C.byref(kv), C.byref(bmap), token_budget, C.byref(plan)),
           "abs_describe_launch")
    return {f: int(getattr(plan, f)) for f, _ in abs_launch_plan._fields_ if f != "reserved"}


def abs_reset_workspace(kv, bmap, token_budget: int, op: int, ws_ptr: int, ws_bytes: int, stream: int) -> None:
    _check(lib().abs_reset_workspace(C.byref(kv), C.byref(bmap), token_budget, op, ws_ptr, ws_bytes, stream),
           "abs_reset_workspace")


def abs_set_debug_checks(enable: bool) -> bool:
    return bool(lib().abs_set_debug_checks(1 if enable else 0))


def abs_head_recall(kv, lse_sel_ptr: int, lse_full_ptr: int, recall_ptr: int, stream: int) -> None:
    _check(lib().abs_head_recall(C.byref(kv), lse_sel_ptr, lse_full_ptr, recall_ptr, stream), "abs_head_recall")


def abs_gather_tiles(tile_addr_ptr: int, num_tiles: int, tile_bytes: int, workgroups: int, in_flight: int,
                     xor_out_ptr: int, stream: int) -> None:
    _check(lib().abs_gather_tiles(tile_addr_ptr, num_tiles, tile_bytes, workgroups, in_flight, xor_out_ptr, stream),
           "abs_gather_tiles")


def abs_assign_block_sizes(recall_host: np.ndarray, threshold: float) -> np.ndarray:
    """recall_host: [3][num_kv_heads] (block sizes 16, 32, 64) -> int32 [num_kv_heads]."""
    r = np.ascontiguousarray(recall_host, dtype=np.float32)
    assert r.ndim == 2 and r.shape[0] == 3
    out = np.zeros(r.shape[1], dtype=np.int32)
    _check(lib().abs_assign_block_sizes(r.shape[1], r.ctypes.data, threshold, out.ctypes.data),
           "abs_assign_block_sizes")
    return out


# ---- torch-side holder ------------------------------------------------------

def _ptr(t) -> int:
    return int(t.data_ptr()) if t is not None else 0


def torch_dtype(kv_dtype: str):
    import torch
    return torch.bfloat16 if kv_dtype == "bf16" else torch.float32


def upload(a: np.ndarray, device, kv_dtype: Optional[str] = None):
    """Host array -> device tensor (bf16 bit patterns become torch.bfloat16)."""
    import torch
    if kv_dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


@dataclass
class PagedKV:
    """One layer's paged cache + block map on the device, with its descriptors."""
    k_cache: object
    v_cache: object
    page_table: object
    seq_lens: object
    seq_lens_host: np.ndarray
    block_size: object
    block_size_host: np.ndarray
    centroid_off: object
    num_q_heads: int
    kv_dtype: str
    kv: abs_paged_kv = field(init=False)
    bmap: abs_block_map = field(init=False)

    def __post_init__(self):
        self.seq_lens_host = np.ascontiguousarray(self.seq_lens_host, dtype=np.int32)
        self.block_size_host = np.ascontiguousarray(self.block_size_host, dtype=np.int32)
        P, Hkv, page, D = self.k_cache.shape
        self.kv = abs_paged_kv(
            num_seqs=len(self.seq_lens_host), num_q_heads=self.num_q_heads, num_kv_heads=Hkv, head_dim=D,
            page_size=page, max_pages_per_seq=self.page_table.shape[1], num_pages=P,
            kv_dtype=ABS_BF16 if self.kv_dtype == "bf16" else ABS_F32, reserved0=0,
            k_cache=_ptr(self.k_cache), v_cache=_ptr(self.v_cache), page_table=_ptr(self.page_table),
            seq_lens=_ptr(self.seq_lens), seq_lens_host=self.seq_lens_host.ctypes.data)
        self.bmap = abs_block_map(block_size_host=self.block_size_host.ctypes.data,
                                  block_size=_ptr(self.block_size), centroid_off=_ptr(self.centroid_off))

    @classmethod
    def from_host(cls, q_heads: int, k_cache: np.ndarray, v_cache: np.ndarray, page_table: np.ndarray,
                  seq_lens: np.ndarray, block_size: np.ndarray, kv_dtype: str, device="cuda",
                  capacity_tokens: Optional[int] = None) -> "PagedKV":
        """capacity_tokens: leave centroid rows for sequences of up to that
        many tokens (abs_centroid_offsets_capacity), for later appends."""
        import torch
        sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
        bs = np.ascontiguousarray(block_size, dtype=np.int32)
        self = cls(upload(k_cache, device, kv_dtype), upload(v_cache, device, kv_dtype),
                   upload(np.ascontiguousarray(page_table, dtype=np.int32), device),
                   upload(sl, device), sl, upload(bs, device), bs,
                   torch.zeros(len(sl) * len(bs) + 1, dtype=torch.int64, device=device), q_heads, kv_dtype)
        off = (abs_centroid_offsets(self.kv, self.bmap) if capacity_tokens is None
               else abs_centroid_offsets_capacity(self.kv, self.bmap, capacity_tokens))
        self.centroid_off.copy_(torch.from_numpy(off))
        self.centroid_rows = int(off[-1])
        return self

    def with_lengths(self, seq_lens: np.ndarray) -> "PagedKV":
        """The same cache, page table and centroid offsets, other sequence
        lengths (tokens appended in place); the offsets must have room."""
        sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
        out = PagedKV(self.k_cache, self.v_cache, self.page_table, upload(sl, self.k_cache.device), sl,
                      self.block_size, self.block_size_host, self.centroid_off, self.num_q_heads, self.kv_dtype)
        out.centroid_rows = self.centroid_rows
        return out

    def with_block_sizes(self, block_size: np.ndarray) -> "PagedKV":
        """The same cache, page table and lengths under another block-size map
        (its own compact centroid offsets)."""
        import torch
        bs = np.ascontiguousarray(block_size, dtype=np.int32)
        dev = self.k_cache.device
        out = PagedKV(self.k_cache, self.v_cache, self.page_table, self.seq_lens, self.seq_lens_host, upload(bs, dev),
                      bs, torch.zeros(len(self.seq_lens_host) * len(bs) + 1, dtype=torch.int64, device=dev),
                      self.num_q_heads, self.kv_dtype)
        off = abs_centroid_offsets(out.kv, out.bmap)
        out.centroid_off.copy_(torch.from_numpy(off))
        out.centroid_rows = int(off[-1])
        return out

    @property
    def head_dim(self) -> int:
        return int(self.kv.head_dim)

    def total_blocks(self) -> int:
        return abs_total_blocks(self.kv, self.bmap)

    def select_capacity(self, budget: int) -> int:
        return abs_select_capacity(self.kv, self.bmap, budget)

    def workspace_bytes(self, budget: int, op: int) -> int:
        return abs_workspace_bytes(self.kv, self.bmap, budget, op)

    def launch_plan(self, budget: int) -> dict:
        return abs_describe_launch(self.kv, self.bmap, budget)


@dataclass
class Centroids:
    codes: object      # uint8 [total_blocks][row bytes]
    scale: object      # f32 [B][Hkv][D]
    lo: object         # f32 [B][Hkv][D]
    fmt: str = "int4"  # a CENTROID_FORMATS name
    desc: abs_centroids = field(init=False)

    def __post_init__(self):
        self.desc = abs_centroids(codes=_ptr(self.codes), scale=_ptr(self.scale), lo=_ptr(self.lo),
                                  format=CENTROID_FORMATS[self.fmt], reserved0=0)

    @classmethod
    def empty(cls, kv: PagedKV, fmt: str = "int4") -> "Centroids":
        import torch
        dev = kv.k_cache.device
        B, Hkv, D = kv.kv.num_seqs, kv.kv.num_kv_heads, kv.kv.head_dim
        rows = getattr(kv, "centroid_rows", None) or kv.total_blocks()
        rb = abs_centroid_row_bytes(D, CENTROID_FORMATS[fmt])
        return cls(torch.zeros(rows, rb, dtype=torch.uint8, device=dev),
                   torch.empty(B, Hkv, D, dtype=torch.float32, device=dev),
                   torch.empty(B, Hkv, D, dtype=torch.float32, device=dev), fmt)


def current_stream() -> int:
    import torch
    return int(torch.cuda.current_stream().cuda_stream)


def workspace(nbytes: int, device="cuda"):
    """Zero-filled device workspace (the decode workspace must start zeroed)."""
    import torch
    return torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def build_centroids(kv: PagedKV, cents: Centroids, ws=None, stream: Optional[int] = None) -> Centroids:
    need = kv.workspace_bytes(1, ABS_OP_BUILD)
    ws = workspace(need, kv.k_cache.device) if ws is None else ws
    abs_build_centroids(kv.kv, kv.bmap, cents.desc, _ptr(ws), ws.numel(),
                        current_stream() if stream is None else stream)
    return cents


def update_centroids(kv: PagedKV, cents: Centroids, appended: int, out_of_range=None,
                     stream: Optional[int] = None) -> None:
    abs_update_centroids(kv.kv, kv.bmap, cents.desc, appended,
                         _ptr(out_of_range) if out_of_range is not None else None,
                         current_stream() if stream is None else stream)


def score_select(kv: PagedKV, cents: Centroids, q, budget: int, sel, count, ws=None,
                 stream: Optional[int] = None) -> None:
    need = kv.workspace_bytes(budget, ABS_OP_SELECT)
    ws = workspace(need, kv.k_cache.device) if ws is None else ws
    abs_score_select(kv.kv, kv.bmap, cents.desc, _ptr(q), budget, _ptr(sel), int(sel.shape[-1]), _ptr(count),
                     _ptr(ws), ws.numel(), current_stream() if stream is None else stream)


def sparse_decode(kv: PagedKV, q, sel, count, budget: int, sm_scale: float, out, lse=None, ws=None,
                  stream: Optional[int] = None) -> None:
    need = kv.workspace_bytes(budget, ABS_OP_DECODE)
    ws = workspace(need, kv.k_cache.device) if ws is None else ws
    abs_sparse_decode(kv.kv, kv.bmap, _ptr(q), _ptr(sel), int(sel.shape[-1]), _ptr(count), budget, sm_scale,
                      _ptr(out), _ptr(lse) if lse is not None else None, _ptr(ws), ws.numel(),
                      current_stream() if stream is None else stream)


def select_decode(kv: PagedKV, cents: Centroids, q, budget: int, sm_scale: float, sel, count, out, lse=None,
                  ws=None, stream: Optional[int] = None) -> None:
    """score_select then sparse_decode through abs_select_decode (fewer launches).
    The call zero-fills the decode's arrival counters itself."""
    need = kv.workspace_bytes(budget, ABS_OP_SELECT_DECODE)
    ws = workspace(need, kv.k_cache.device) if ws is None else ws
    abs_select_decode(kv.kv, kv.bmap, cents.desc, _ptr(q), budget, sm_scale, _ptr(sel), int(sel.shape[-1]),
                      _ptr(count), _ptr(out), _ptr(lse) if lse is not None else None, _ptr(ws), ws.numel(),
                      current_stream() if stream is None else stream)


CALIBRATION_SIZES = (16, 32, 64)


def calibrate_block_sizes(kv: PagedKV, q, budget: int, sm_scale: float, threshold: float = 0.95,
                          fmt: str = "int4", stream: Optional[int] = None):
    """Offline calibration of the per-head block-size map on one layer (see
    abs_head_recall / abs_assign_block_sizes): for each block size, the
    layer with that size everywhere is built, selected and decoded; the
    decode with every block selected gives the full normalizers.  Returns
    (block sizes int32 [Hkv], recall fp32 [3][Hkv]).  Synchronizes once, to
    read the recalls."""
    import torch
    dev = kv.k_cache.device
    st = current_stream() if stream is None else stream
    B, Hq, Hkv = kv.kv.num_seqs, kv.kv.num_q_heads, kv.kv.num_kv_heads
    D = kv.kv.head_dim
    out = torch.empty((B, Hq, D), dtype=torch_dtype(kv.kv_dtype), device=dev)
    lse_full = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    lse_sel = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    recall = torch.empty((3, Hkv), dtype=torch.float32, device=dev)
    everything = int(kv.seq_lens_host.max())

    def select_and_decode(layer, cents, bud, lse):
        cap = layer.select_capacity(bud)
        sel = torch.empty((B, Hkv, cap), dtype=torch.int32, device=dev)
        cnt = torch.empty((B, Hkv), dtype=torch.int32, device=dev)
        score_select(layer, cents, q, bud, sel, cnt, stream=st)
        sparse_decode(layer, q, sel, cnt, bud, sm_scale, out, lse, stream=st)

    for k, bs in enumerate(CALIBRATION_SIZES):
        layer = kv.with_block_sizes(np.full(Hkv, bs, dtype=np.int32))
        cents = build_centroids(layer, Centroids.empty(layer, fmt), stream=st)
        if k == 0:
            select_and_decode(layer, cents, everything, lse_full)
        select_and_decode(layer, cents, budget, lse_sel)
        abs_head_recall(layer.kv, _ptr(lse_sel), _ptr(lse_full), _ptr(recall[k]), st)
    torch.cuda.synchronize(dev)
    r = recall.cpu().numpy()
    return abs_assign_block_sizes(r, threshold), r
