"""Shared helpers for the GPU parity tests: move a seeded workload to the
device and compare results with the oracle at the stated tolerances."""

from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import paged_kv_cache_resolve_amd as pk

# Attention tolerances: fp32 max-abs 1e-4; bf16 |gpu - ref| <= 2e-2 + 2e-2 |ref|
# (both as stated for the method).  fp16 (no stated tolerance) is derived
# from the arithmetic, per (sequence, query head) with vmax = max |V| over the
# rows it attends:
#   - each probability is rounded to fp16 (relative error u = 2^-11; the
#     2^15 pre-scale keeps weights down to 2^-29 normal) and the normaliser
#     sums the rounded values, so the output is an exact convex combination
#     of V rows whose weights are off by a factor (1+d)/(1+e), |d|, |e| <= u:
#     at most 2u/(1-u) vmax <= 2^-10 (1 + 2^-10) vmax;
#   - the fp16 output rounding adds 2^-11 |out| <= 2^-11 (1 + 2^-10) |ref|;
#   - fp32 accumulation of the products and sums is allowed 2^-14 vmax
#     (an allowance, not a worst-case bound; measured errors sit far below).
F32_ATOL = 1e-4
BF16_ATOL = 2e-2
BF16_RTOL = 2e-2
F16_VMAX_FACTOR = 2.0**-10 * (1 + 2.0**-10) + 2.0**-14
F16_RTOL = 2.0**-11 * (1 + 2.0**-10)
NAN_BITS = {"f32": np.float32(np.nan), "bf16": np.uint16(0x7FC0), "f16": np.float16(np.nan)}


def say(msg: str) -> None:
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def t_dtype(dtype: str):
    return {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[dtype]


def np_to_dev(x: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    """float32 / float16 array or bf16 bit patterns (uint16) -> device tensor."""
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)
    if dtype == "f16":
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float16)).to(device)
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.uint16).view(np.int16))
    return t.to(device).view(torch.bfloat16)


def dev_to_np(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> float32 / float16 array or bf16 bit patterns (uint16)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def dev_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


class DeviceWorkload:
    """A Workload's arrays on the GPU plus a pool handle over them."""

    def __init__(self, w, device="cuda"):
        self.w = w
        data = np_to_dev(w.pool, w.dtype, device)
        self.pool = pk.KVPool(w.NB, w.BS, w.L, w.Hkv, w.D, t_dtype(w.dtype), data=data)
        self.tables = torch.from_numpy(w.block_tables).to(device)
        self.lens = torch.from_numpy(w.context_lens).to(device)
        self.positions = torch.from_numpy(w.positions).to(device)
        # the preconditions the library trusts, checked on the host copy
        pk.validate_decode_inputs(w.NB, w.BS, self.tables, self.lens)
        self.q = np_to_dev(w.q, w.dtype, device)
        self.k_new = np_to_dev(w.k_new, w.dtype, device)
        self.v_new = np_to_dev(w.v_new, w.dtype, device)

    def decode(self, out=None):
        if out is None:
            out = torch.empty_like(self.q)
        pk.paged_attention_decode(out, self.q, self.pool, self.w.layer, self.tables, self.lens,
                                  self.w.scale)
        return out


def attended_vmax(pool: np.ndarray, dtype: str, layer: int, block_tables: np.ndarray,
                  context_lens: np.ndarray, num_q_heads: int, rows=None):
    """[S, num_q_heads] max |V| over the cached rows each (sequence, query
    head) attends (0 where T_b = 0), from the host pool through the oracle's
    gather; the scale of the fp16 tolerance.  None for other dtypes."""
    if dtype != "f16":
        return None
    S = len(context_lens)
    hkv = pool.shape[3]
    G = num_q_heads // hkv
    out = np.zeros((S, num_q_heads))
    for b in (range(S) if rows is None else rows):
        T = int(context_lens[b])
        if T == 0:
            continue
        _, V = oracle.gather_sequence(pool, layer, block_tables[b], T)
        out[b] = np.repeat(np.abs(oracle.widen(V, dtype)).max(axis=(0, 2)), G)
    return out


def dense_vmax(v: np.ndarray, mask: np.ndarray, dtype: str, num_q_heads: int):
    """attended_vmax of a gathered, padded batch: v [S, max_len, Hkv, D],
    token t of sequence b attended where mask[b, t] != 0."""
    if dtype != "f16":
        return None
    S, _, hkv, _ = v.shape
    a = np.abs(oracle.widen(v, dtype)).max(axis=3)              # [S, max_len, Hkv]
    a = np.where(mask[:, :, None] != 0, a, 0.0).max(axis=1) if v.shape[1] else np.zeros((S, hkv))
    return np.repeat(a, num_q_heads // hkv, axis=1)


def workload_vmax(w, pool=None, rows=None):
    """attended_vmax of a Workload (optionally over another host pool)."""
    return attended_vmax(w.pool if pool is None else pool, w.dtype, w.layer, w.block_tables,
                         w.context_lens, w.Hq, rows)


def assert_attention_close(gpu: torch.Tensor, ref: np.ndarray, dtype: str, rows=None, what="",
                           vmax=None):
    """fp32: max-abs 1e-4; bf16: |gpu - ref| <= 2e-2 + 2e-2 |ref|; fp16:
    |gpu - ref| <= F16_VMAX_FACTOR * vmax[b, h] + F16_RTOL |ref| with vmax
    the [S, Hq] attended max |V| (required for fp16)."""
    g = dev_to_f64(gpu)
    if rows is not None:
        g, ref = g[rows], ref[rows]
        if vmax is not None:
            vmax = vmax[rows]
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    err = np.abs(g - ref)
    if dtype == "f32":
        worst = float(err.max()) if err.size else 0.0
        assert worst <= F32_ATOL, f"{what}: max abs err {worst:.3e} > {F32_ATOL}"
    else:
        if dtype == "f16":
            assert vmax is not None, f"{what}: the fp16 bound needs the attended max |V|"
            bound = F16_VMAX_FACTOR * vmax[:, :, None] + F16_RTOL * np.abs(ref)
        else:
            bound = BF16_ATOL + BF16_RTOL * np.abs(ref)
        bad = err > bound
        assert not bad.any(), (f"{what}: {int(bad.sum())} elements out of tolerance, "
                               f"worst excess {float((err - bound).max()):.3e}")
    return float(err.max()) if err.size else 0.0
