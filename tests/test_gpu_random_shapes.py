"""Seeded random shapes against the oracle, under both decode splits.

Each case draws a dtype, head_dim, KV heads, query heads per KV head, block
size, batch and a mix of context lengths (empty, short, long), so that the
cases between them reach every pass-1 form (16-bit and fp32 MFMA streams, the
VALU kernel, 4- and 8-token blocks, virtual KV heads, the per-pair kernel and
the chunk split with its merge).  The plain decode is compared with the
oracle's; the fused step also against the oracle's append, bit for bit.
"""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_resolve_amd as pk
from workloads import make_workload

from gpu_helpers import (NAN_BITS, DeviceWorkload, assert_attention_close, dev_to_np, np_to_dev, say,
                         workload_vmax)

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU"),
]

HEAD_DIMS = {"bf16": [64, 96, 128, 256, 40, 200], "f16": [64, 96, 128, 256, 40, 200],
             "f32": [64, 128, 96, 36, 100, 256]}


def draw_cases(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        dtype = ["bf16", "f16", "f32"][rng.integers(3)]
        D = int(rng.choice(HEAD_DIMS[dtype]))
        Hkv = int(rng.choice([1, 2, 4, 8]))
        G = int(rng.choice([1, 2, 3, 4, 5, 7, 8, 12, 16, 17, 24, 32]))
        while G * Hkv > 64:
            Hkv //= 2
        BS = int(rng.choice([1, 2, 4, 8, 16, 32, 64]))
        S = int(rng.integers(1, 21))
        top = int(rng.choice([64, 256, 1200]))
        kind = rng.random(S)
        lens = np.where(kind < 0.1, 0,
                        np.where(kind < 0.4, rng.integers(1, 65, S), rng.integers(1, top + 1, S)))
        cases.append((i, dtype, G * Hkv, Hkv, D, BS, [int(t) for t in lens]))
    return cases


CASES = draw_cases(40, 20261203)


def build(dtype, Hq, Hkv, D, BS, lens, extra_block=False):
    lens = np.asarray(lens, dtype=np.int32)
    mb = max(1, max(math.ceil(int(t) / BS) for t in lens)) + (1 if extra_block else 0)
    nb = sum(math.ceil(int(t) / BS) for t in lens) + len(lens) + 3
    return make_workload(0, dtype=dtype, S=len(lens), Hq=Hq, Hkv=Hkv, D=D, BS=BS, L=2, layer=1,
                         context_lens=lens, MB=mb, NB=nb, tables="perm")


def split_id(split):
    return pk.SPLIT_AUTO if split == "auto" else pk.SPLIT_CHUNKS


@pytest.mark.parametrize("split", ["auto", "chunks"])
@pytest.mark.parametrize("i,dtype,Hq,Hkv,D,BS,lens", CASES, ids=[f"case{c[0]}" for c in CASES])
def test_random_shape_decode(i, dtype, Hq, Hkv, D, BS, lens, split):
    say(f"random case {i}: {dtype} Hq={Hq} Hkv={Hkv} D={D} BS={BS} S={len(lens)} "
        f"max T={max(lens)} split={split}")
    w = build(dtype, Hq, Hkv, D, BS, lens)
    # NaN in every slot no sequence owns
    slots = oracle.resolve_slots(w.block_tables, w.context_lens, w.BS, max(w.max_len, 1))
    used = np.zeros(w.NB * w.BS, dtype=bool)
    used[slots[slots >= 0]] = True
    blk, off = np.nonzero(~used.reshape(w.NB, w.BS))
    w.pool[blk, :, :, :, off, :] = NAN_BITS[w.dtype]
    dw = DeviceWorkload(w)
    with pk.split_mode(split_id(split)):
        out = dw.decode()
        torch.cuda.synchronize()
    ref = oracle.paged_attention_decode(w.pool, w.dtype, w.layer, w.block_tables,
                                        w.context_lens, w.q, w.scale)
    assert_attention_close(out, ref, dtype, what=f"random case {i}", vmax=workload_vmax(w))
    empty = [b for b, t in enumerate(lens) if t == 0]
    assert not dev_to_np(out)[empty].any(), "empty sequences must give zero rows"


@pytest.mark.parametrize("split", ["auto", "chunks"])
@pytest.mark.parametrize("i,dtype,Hq,Hkv,D,BS,lens", CASES[:16], ids=[f"case{c[0]}" for c in CASES[:16]])
def test_random_shape_fused_step(i, dtype, Hq, Hkv, D, BS, lens, split):
    """The decode step with the new token at position T_b - 1 (none for an
    empty sequence): output against the oracle, pool bit for bit against the
    oracle's append."""
    say(f"random fused case {i}: {dtype} Hq={Hq} Hkv={Hkv} D={D} BS={BS} S={len(lens)} "
        f"split={split}")
    w = build(dtype, Hq, Hkv, D, BS, lens)
    positions = [t - 1 for t in lens]   # -1 for an empty sequence: no token
    for b, pos in enumerate(positions):
        if pos >= 0:
            w.pool[w.block_tables[b, pos // BS], :, w.layer, :, pos % BS, :] = NAN_BITS[dtype]
    dw = DeviceWorkload(w)
    out = torch.empty_like(dw.q)
    pos_t = torch.from_numpy(np.asarray(positions, np.int32)).cuda()
    with pk.split_mode(split_id(split)):
        pk.paged_attention_decode_append(out, dw.q, dw.pool, w.layer, dw.tables, dw.lens, w.scale,
                                         dw.k_new, dw.v_new, pos_t)
        torch.cuda.synchronize()
    ref_pool = oracle.kv_append(w.pool, w.layer, w.block_tables, positions, w.k_new, w.v_new)
    ref = oracle.paged_attention_decode(ref_pool, w.dtype, w.layer, w.block_tables,
                                        w.context_lens, w.q, w.scale)
    assert_attention_close(out, ref, dtype, what=f"random fused case {i}",
                           vmax=workload_vmax(w, pool=ref_pool))
    assert dev_to_np(dw.pool.data).tobytes() == ref_pool.tobytes(), "pool differs from oracle append"


def random_rows(rng, shape, dtype):
    """Random rows in the pool's storage format (bf16 as bit patterns)."""
    x = rng.standard_normal(shape, dtype=np.float32)
    if dtype == "bf16":
        from workloads import bf16_round_bits
        return bf16_round_bits(x)
    return x.astype(np.float16) if dtype == "f16" else x


@pytest.mark.parametrize("i,dtype,Hq,Hkv,D,BS,lens", CASES[:16], ids=[f"case{c[0]}" for c in CASES[:16]])
def test_random_shape_gather(i, dtype, Hq, Hkv, D, BS, lens):
    """paged_kv_gather against the oracle's gather, bit for bit, with a
    max_len past the longest sequence (all-padding tail)."""
    say(f"random gather case {i}: {dtype} Hkv={Hkv} D={D} BS={BS} S={len(lens)}")
    w = build(dtype, Hq, Hkv, D, BS, lens)
    dw = DeviceWorkload(w)
    max_len = max(lens) + 5
    k, v, mask = pk.paged_kv_gather(dw.pool, w.layer, dw.tables, dw.lens, max_len)
    torch.cuda.synchronize()
    rk, rv, rm = oracle.paged_kv_gather(w.pool, w.layer, w.block_tables, w.context_lens, max_len)
    assert dev_to_np(k).tobytes() == rk.tobytes()
    assert dev_to_np(v).tobytes() == rv.tobytes()
    assert mask.cpu().numpy().tobytes() == rm.tobytes()


@pytest.mark.parametrize("i,dtype,Hq,Hkv,D,BS,lens", CASES[:16], ids=[f"case{c[0]}" for c in CASES[:16]])
def test_random_shape_appends(i, dtype, Hq, Hkv, D, BS, lens):
    """kv_append_tokens (a ragged run of tokens per sequence, some skipped)
    and kv_append_layers (one token on every layer) against the oracle's
    appends: the whole pool, bit for bit."""
    say(f"random appends case {i}: {dtype} Hkv={Hkv} D={D} BS={BS} S={len(lens)}")
    w = build(dtype, Hq, Hkv, D, BS, lens)
    rng = np.random.default_rng(1000 + i)
    S = len(lens)
    starts = np.full(S, -1, dtype=np.int32)
    counts = np.zeros(S, dtype=np.int32)
    for b, T in enumerate(lens):
        if T > 0 and rng.random() < 0.85:
            starts[b] = rng.integers(0, T)
            counts[b] = rng.integers(1, T - starts[b] + 1)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    total = int(offsets[-1])
    kr = random_rows(rng, (total, Hkv, D), dtype)
    vr = random_rows(rng, (total, Hkv, D), dtype)
    dw = DeviceWorkload(w)
    if total > 0:
        pk.kv_append_tokens(dw.pool, w.layer, np_to_dev(kr, dtype), np_to_dev(vr, dtype),
                            dw.tables, torch.from_numpy(starts).cuda(),
                            torch.from_numpy(offsets).cuda())
    positions = np.array([t - 1 for t in lens], dtype=np.int32)
    kl = random_rows(rng, (S, w.L, Hkv, D), dtype)
    vl = random_rows(rng, (S, w.L, Hkv, D), dtype)
    pk.kv_append_layers(dw.pool, np_to_dev(kl, dtype), np_to_dev(vl, dtype), dw.tables,
                        torch.from_numpy(positions).cuda())
    torch.cuda.synchronize()
    ref = oracle.kv_append_tokens(w.pool, w.layer, w.block_tables, starts, offsets, kr, vr)
    ref = oracle.kv_append_layers(ref, w.block_tables, positions, kl, vl)
    assert dev_to_np(dw.pool.data).tobytes() == ref.tobytes(), "pool differs from the oracle's appends"


DENSE_CASES = [c for c in CASES if c[1] != "f32" and c[4] in (64, 96, 128, 256)][:12]


@pytest.mark.parametrize("i,dtype,Hq,Hkv,D,BS,lens", DENSE_CASES,
                         ids=[f"case{c[0]}" for c in DENSE_CASES])
def test_random_shape_gather_then_dense(i, dtype, Hq, Hkv, D, BS, lens):
    """The gather-then-attend path (paged_kv_gather, then
    dense_attention_decode over the padded batch) against the oracle's paged
    decode of the same pool: the padding and the mask must leave the result
    unchanged."""
    say(f"random gather+dense case {i}: {dtype} Hq={Hq} Hkv={Hkv} D={D} BS={BS} S={len(lens)}")
    w = build(dtype, Hq, Hkv, D, BS, lens)
    dw = DeviceWorkload(w)
    k, v, mask = pk.paged_kv_gather(dw.pool, w.layer, dw.tables, dw.lens, max(lens) + 3)
    out = torch.empty_like(dw.q)
    pk.dense_attention_decode(out, dw.q, k, v, mask, w.scale)
    torch.cuda.synchronize()
    ref = oracle.paged_attention_decode(w.pool, w.dtype, w.layer, w.block_tables,
                                        w.context_lens, w.q, w.scale)
    assert_attention_close(out, ref, dtype, what=f"gather+dense case {i}", vmax=workload_vmax(w))
