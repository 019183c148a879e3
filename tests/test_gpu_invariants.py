"""Exact invariants of attention, checked on the GPU's own outputs (no
oracle value involved): outputs lie in the convex hull of the attended V
rows, a constant shift of every K row changes nothing, a constant shift of
every V row shifts the output, identical sequences give identical outputs,
and the result does not depend on how the chunk space is split between
wavefronts (a sequence alone or inside a large batch)."""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
from workloads import make_workload

from gpu_helpers import DeviceWorkload, dev_to_f64, say

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU"),
]

SLACK = {"f32": 1e-6, "bf16": 2.0 ** -8, "f16": 2.0 ** -11}   # output rounding, relative


def custom(dtype, S, Hq, Hkv, D, BS, lens, seed_offset=0):
    lens = np.asarray(lens, dtype=np.int32)
    mb = max(1, max(math.ceil(int(t) / BS) for t in lens))
    nb = sum(math.ceil(int(t) / BS) for t in lens) + 3
    return make_workload(0, dtype=dtype, S=S, Hq=Hq, Hkv=Hkv, D=D, BS=BS, L=1, layer=0,
                         context_lens=lens, MB=mb, NB=nb, tables="perm", seed_offset=seed_offset)


def rows_of(w, b):
    """(block, offset) of every cached token of sequence b."""
    return [(int(w.block_tables[b, t // w.BS]), t % w.BS) for t in range(int(w.context_lens[b]))]


@pytest.mark.parametrize("dtype,Hq,Hkv,D,BS", [("bf16", 32, 8, 128, 16), ("f16", 14, 2, 64, 32),
                                               ("f32", 8, 2, 128, 16), ("bf16", 6, 2, 96, 16)])
def test_output_in_convex_hull_of_v(dtype, Hq, Hkv, D, BS, split):
    say(f"convex hull {dtype} D={D}")
    w = custom(dtype, 6, Hq, Hkv, D, BS, [1, 17, 300, 2000, 33, 64])
    out = dev_to_f64(DeviceWorkload(w).decode())
    G = Hq // Hkv
    for b in range(w.S):
        _, V = oracle.gather_sequence(w.pool, 0, w.block_tables[b], int(w.context_lens[b]))
        V = oracle.widen(V, dtype)
        for h in range(Hq):
            lo, hi = V[:, h // G, :].min(axis=0), V[:, h // G, :].max(axis=0)
            slack = SLACK[dtype] * np.maximum(np.abs(lo), np.abs(hi))
            assert (out[b, h] >= lo - slack).all() and (out[b, h] <= hi + slack).all(), (b, h)


def _shift_rows(w, kv, shift):
    """Add shift[g] to the K (kv = 0) or V (kv = 1) rows of every cached token."""
    for b in range(w.S):
        for blk, off in rows_of(w, b):
            w.pool[blk, kv, 0, :, off, :] += shift


@pytest.mark.parametrize("D,BS", [(128, 16), (64, 32), (96, 16)])
def test_k_shift_invariance_and_v_shift_equivariance(D, BS, split):
    """fp32 pools, so that the shifted values are exact inputs."""
    say(f"K/V shift D={D} BS={BS}")
    lens = [5, 100, 1500, 37, 16]
    base = custom("f32", 5, 8, 2, D, BS, lens)
    ref = dev_to_f64(DeviceWorkload(base).decode())
    rng = np.random.default_rng(D)
    c = rng.standard_normal((2, D)).astype(np.float32)
    wk = custom("f32", 5, 8, 2, D, BS, lens)
    _shift_rows(wk, 0, c)
    out_k = dev_to_f64(DeviceWorkload(wk).decode())
    assert np.abs(out_k - ref).max() <= 1e-4
    wv = custom("f32", 5, 8, 2, D, BS, lens)
    _shift_rows(wv, 1, c)
    out_v = dev_to_f64(DeviceWorkload(wv).decode())
    G = 4
    want = ref + np.repeat(c.astype(np.float64), G, axis=0)[None, :, :]
    assert np.abs(out_v - want).max() <= 1e-4


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_identical_sequences_identical_outputs(dtype, split):
    """Sequence 4 gets sequence 1's K/V rows (in its own blocks) and its q."""
    say(f"identical sequences {dtype}")
    lens = [40, 3000, 7, 900, 3000, 1]
    w = custom(dtype, 6, 16, 4, 128, 16, lens)
    for (b1, o1), (b4, o4) in zip(rows_of(w, 1), rows_of(w, 4)):
        w.pool[b4, :, 0, :, o4, :] = w.pool[b1, :, 0, :, o1, :]
    w.q[4] = w.q[1]
    out = dev_to_f64(DeviceWorkload(w).decode())
    tol = 1e-6 if dtype == "f32" else 2.0 ** -7 * np.abs(out[1]).max()
    assert np.abs(out[1] - out[4]).max() <= tol


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_split_independence(dtype):
    """One long sequence alone (its chunks spread over every wavefront) and
    the same sequence inside a batch of 64 (a few wavefronts each) agree."""
    say(f"split independence {dtype}")
    alone = custom(dtype, 1, 32, 8, 128, 16, [20000])
    a = dev_to_f64(DeviceWorkload(alone).decode())[0]
    rng = np.random.default_rng(9)
    lens = rng.integers(500, 1500, size=64)
    lens[17] = 20000
    batch = custom(dtype, 64, 32, 8, 128, 16, lens)
    blocks = rows_of(alone, 0)
    for (bs, os_), (bd, od) in zip(blocks, rows_of(batch, 17)):
        batch.pool[bd, :, 0, :, od, :] = alone.pool[bs, :, 0, :, os_, :]
    batch.q[17] = alone.q[0]
    b = dev_to_f64(DeviceWorkload(batch).decode())[17]
    tol = 1e-5 if dtype == "f32" else 2.0 ** -7 * np.abs(a).max()
    assert np.abs(a - b).max() <= tol
