"""Shared helpers for the GPU parity tests: move a seeded workload to the
device and compare results with the oracle at the stated tolerances."""

from __future__ import annotations

import sys

import numpy as np
import torch

import paged_kv_cache_resolve_amd as pk

# Attention tolerances: fp32 max-abs 1e-4; bf16 |gpu - ref| <= 2e-2 + 2e-2 |ref|;
# fp16 |gpu - ref| <= 5e-3 + 5e-3 |ref| (derived from the arithmetic: weights
# rounded to fp16 move a convex combination of V rows by at most 2^-10 max|V|,
# and the output rounding is 2^-11 |out|).
F32_ATOL = 1e-4
BF16_ATOL = 2e-2
BF16_RTOL = 2e-2
F16_ATOL = 5e-3
F16_RTOL = 5e-3
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


def assert_attention_close(gpu: torch.Tensor, ref: np.ndarray, dtype: str, rows=None, what=""):
    g = dev_to_f64(gpu)
    if rows is not None:
        g, ref = g[rows], ref[rows]
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    err = np.abs(g - ref)
    if dtype == "f32":
        worst = float(err.max()) if err.size else 0.0
        assert worst <= F32_ATOL, f"{what}: max abs err {worst:.3e} > {F32_ATOL}"
    else:
        atol, rtol = (F16_ATOL, F16_RTOL) if dtype == "f16" else (BF16_ATOL, BF16_RTOL)
        bound = atol + rtol * np.abs(ref)
        bad = err > bound
        assert not bad.any(), (f"{what}: {int(bad.sum())} elements out of tolerance, "
                               f"worst excess {float((err - bound).max()):.3e}")
    return float(err.max()) if err.size else 0.0
