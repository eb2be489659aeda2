"""Run the HIP path through the C ABI on one layer of inputs and bring the
results back to the host, plus the comparison rules the parity tests use.

Comparison rules (how the tolerances are applied):
  * centroid build: codes (every format), scale and lo are compared bit for bit (the
    kernel sums keys in fp64, so its fp32 centroid is the same correctly
    rounded mean as the oracle's, and the quantizer's fp32 steps are the same
    IEEE operations);
  * selection: per (b, h) the selected index sets must be equal, except for
    blocks whose oracle score lies within the tie band of the K-th score tau:
    band = max(1e-4 |tau|, 1e-6 M), M = sum_d |qbar_d| max(|lo_d|, |hi_d|)
    (or, for any centroid format, sum_d |qbar_d| max_j |c_hat_{j,d}|)
    bounds every |score| of the head; indices ascending, K entries;
  * attention: element-wise against the oracle run on the GPU's own
    selection; bf16 max-abs <= 2e-2 and mean-abs <= 2e-3, fp32 max-abs <= 1e-4
    and mean-abs <= 1e-5; lse to 1e-3 (bf16) / 1e-5 (fp32) absolute.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from block_sparse_attention_abs_amd import abs as A
from block_sparse_attention_abs_amd import workload as W

TOL = {"bf16": dict(max_abs=2e-2, mean_abs=2e-3, lse=1e-3), "f32": dict(max_abs=1e-4, mean_abs=1e-5, lse=1e-5)}


@dataclass
class GpuResult:
    codes: np.ndarray     # uint8 [total][D] unpacked (0..15)
    scale: np.ndarray
    lo: np.ndarray
    sel: np.ndarray       # int32 [B][Hkv][cap]
    count: np.ndarray
    out: np.ndarray       # fp32 [B][Hq][D]
    lse: np.ndarray


def unpack_codes(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty((p.shape[0], p.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = p & 15
    out[:, 1::2] = p >> 4
    return out


def codes_of_format(raw: np.ndarray, fmt: str) -> np.ndarray:
    """Device code rows (uint8 [rows][row bytes]) -> uint16 [rows][D] code
    values in the layout of abs_centroids."""
    raw = np.ascontiguousarray(raw, dtype=np.uint8)
    if fmt == "bf16":
        return raw.view("<u2").astype(np.uint16)
    if fmt == "int8":
        return raw.astype(np.uint16)
    return unpack_codes(raw).astype(np.uint16)


def pack_codes(codes: np.ndarray) -> np.ndarray:
    c = np.asarray(codes, dtype=np.uint8)
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def to_host_f32(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy()


class GpuLayer:
    """Device copies of one layer's inputs and the ABI descriptors over them."""

    def __init__(self, x: W.LayerInputs, device="cuda"):
        self.x = x
        self.kv = A.PagedKV.from_host(x.q.shape[1], x.k_cache, x.v_cache, x.page_table, x.seq_lens, x.block_size,
                                      x.dtype, device)
        self.q = A.upload(x.q, device, x.dtype)
        self.cents = A.Centroids.empty(self.kv)
        self.device = device

    def build(self):
        A.build_centroids(self.kv, self.cents)
        return self.cents

    def select(self, budget: int, cents: A.Centroids | None = None):
        cap = self.kv.select_capacity(budget)
        B, Hkv = self.x.page_table.shape[0], self.x.k_cache.shape[1]
        sel = torch.full((B, Hkv, cap), -1, dtype=torch.int32, device=self.device)
        cnt = torch.zeros((B, Hkv), dtype=torch.int32, device=self.device)
        A.score_select(self.kv, self.cents if cents is None else cents, self.q, budget, sel, cnt)
        return sel, cnt

    def decode(self, sel, cnt, budget: int, sm_scale: float):
        B, Hq, D = self.x.q.shape
        out = torch.empty((B, Hq, D), dtype=A.torch_dtype(self.x.dtype), device=self.device)
        lse = torch.empty((B, Hq), dtype=torch.float32, device=self.device)
        A.sparse_decode(self.kv, self.q, sel, cnt, budget, sm_scale, out, lse)
        return out, lse

    def run(self, budget: int, sm_scale: float) -> GpuResult:
        self.build()
        sel, cnt = self.select(budget)
        out, lse = self.decode(sel, cnt, budget, sm_scale)
        torch.cuda.synchronize()
        return GpuResult(unpack_codes(self.cents.codes.cpu().numpy()), self.cents.scale.cpu().numpy(),
                         self.cents.lo.cpu().numpy(), sel.cpu().numpy(), cnt.cpu().numpy(), to_host_f32(out),
                         lse.cpu().numpy())


def default_scale(D: int) -> float:
    return float(np.float32(1.0 / np.sqrt(D)))


def check_selection(oracle_mod, x, quant, scores, gpu_sel, gpu_cnt, budget):
    """Selection rule (see module doc).  Returns the number of tie-band swaps."""
    qf = W.to_f32(x.q, x.dtype).astype(np.float64)
    G = x.q.shape[1] // x.k_cache.shape[1]
    swaps = 0
    for b, h, r0, n in oracle_mod.block_rows(x.seq_lens, x.block_size):
        k = oracle_mod.k_of(x.seq_lens[b], x.block_size[h], budget)
        assert gpu_cnt[b, h] == k, (b, h, gpu_cnt[b, h], k)
        got = gpu_sel[b, h, :k]
        assert (np.diff(got) > 0).all() and got.min() >= 0 and got.max() < n, (b, h)
        s = scores[r0:r0 + n]
        order = np.lexsort((np.arange(n), -s))
        want = np.sort(order[:k])
        if np.array_equal(got, want):
            continue
        tau = s[order[k - 1]]
        qbar = qf[b, h * G:(h + 1) * G].sum(0)
        if getattr(quant, "deq", None) is not None:   # any centroid format: bound from the dequantized rows
            M = np.sum(np.abs(qbar) * np.abs(quant.deq[r0:r0 + n]).max(axis=0))
        else:
            hi = quant.lo[b, h].astype(np.float64) + 15 * quant.scale[b, h].astype(np.float64)
            M = np.sum(np.abs(qbar) * np.maximum(np.abs(quant.lo[b, h]), np.abs(hi)))
        band = max(1e-4 * abs(tau), 1e-6 * M)
        diff = np.setxor1d(got, want)
        assert (np.abs(s[diff] - tau) <= band).all(), (b, h, diff, s[diff], tau, band)
        swaps += len(diff) // 2
    return swaps


def check_attention(out, lse, ref_out, ref_lse, dtype):
    t = TOL[dtype]
    err = np.abs(out.astype(np.float64) - ref_out)
    assert err.max() <= t["max_abs"], err.max()
    assert err.mean() <= t["mean_abs"], err.mean()
    assert np.abs(lse.astype(np.float64) - ref_lse).max() <= t["lse"], np.abs(lse - ref_lse).max()
    return float(err.max()), float(err.mean())


def attention_vs_own_selection(out, ref) -> str:
    """Max and mean |out - oracle output over the oracle's own selection|
    (reported, not asserted: a tie-band swap legitimately moves it)."""
    d = np.abs(np.asarray(out, dtype=np.float64) - ref.out)
    return f"max {d.max():.2e} mean {d.mean():.2e}"


def oracle_quant_from_gpu(oracle_mod, g: GpuResult):
    return oracle_mod.Quantized(g.codes, g.scale, g.lo)
