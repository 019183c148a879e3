"""GPU parity of the fused decode step (paged_attention_decode_append): the
output against the oracle's append-then-decode, the whole pool bit-exact
against the oracle's append, and the output bit-identical to the two-call
form (kv_append, then paged_attention_decode).

The pool slot each new token goes to is filled with NaN before the call, so
a decode that read the stale pool row instead of the new token would fail.
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



def poison_append_slots(w, positions):
    """NaN into the layer's K and V rows at every target slot."""
    for b, pos in enumerate(positions):
        if pos < 0:
            continue
        blk = w.block_tables[b, pos // w.BS]
        w.pool[blk, :, w.layer, :, pos % w.BS, :] = NAN_BITS[w.dtype]
    return w


def run_fused(dw, positions):
    w = dw.w
    out = torch.empty_like(dw.q)
    pos = torch.from_numpy(np.asarray(positions, np.int32)).cuda()
    pk.paged_attention_decode_append(out, dw.q, dw.pool, w.layer, dw.tables, dw.lens, w.scale,
                                     dw.k_new, dw.v_new, pos)
    torch.cuda.synchronize()
    return out


def oracle_step(w, positions):
    pool = oracle.kv_append(w.pool, w.layer, w.block_tables, positions, w.k_new, w.v_new)
    ref = oracle.paged_attention_decode(pool, w.dtype, w.layer, w.block_tables, w.context_lens,
                                        w.q, w.scale)
    return pool, ref


def custom(dtype, S, Hq, Hkv, D, BS, lens, positions, L=1, layer=0):
    """A workload with one extra table column, and a spare block placed in
    the table wherever a position lies past the sequence's used blocks (the
    caller's job before an append that opens a new block)."""
    lens = np.asarray(lens, dtype=np.int32)
    mb = max(1, max(math.ceil(int(t) / BS) for t in lens)) + 1
    nb = sum(math.ceil(int(t) / BS) for t in lens) + S + 2
    w = make_workload(0, dtype=dtype, S=S, Hq=Hq, Hkv=Hkv, D=D, BS=BS, L=L, layer=layer,
                      context_lens=lens, MB=mb, NB=nb, tables="perm")
    spare = sorted(set(range(nb)) - set(w.block_tables[w.block_tables >= 0].tolist()))
    for b, pos in enumerate(positions):
        if pos >= 0 and w.block_tables[b, pos // BS] < 0:
            w.block_tables[b, pos // BS] = spare.pop()
    return w


@pytest.mark.parametrize("idx,S", [(0, None), (1, None), (2, 6), (3, 2), (4, 24)])
def test_fused_step_named_workloads(idx, S, split):
    say(f"fused append+decode workload {idx} S={S}")
    w = make_workload(idx, **({"S": S} if S else {}))
    positions = w.positions.copy()
    poison_append_slots(w, positions)
    dw = DeviceWorkload(w)
    out = run_fused(dw, positions)
    ref_pool, ref = oracle_step(w, positions)
    assert_attention_close(out, ref, w.dtype, what=f"fused w{idx}",
                           vmax=workload_vmax(w, pool=ref_pool))
    assert dev_to_np(dw.pool.data).tobytes() == ref_pool.tobytes(), "pool differs from oracle append"


# MFMA shapes (bf16, D 64/128, BS multiple of 16) read the new rows from
# k_new / v_new; the rest take the append launch then the VALU decode.
SHAPES = [
    ("bf16", 8, 2, 128, 16),
    ("bf16", 14, 2, 64, 32),
    ("f16", 14, 2, 64, 16),     # small batches here take the LDS-staged per-pair stream
    ("bf16", 7, 1, 64, 48),     # the same with 48-token blocks
    ("bf16", 16, 1, 128, 16),
    ("bf16", 8, 2, 64, 8),
    ("f32", 8, 2, 64, 16),
    ("f32", 8, 2, 128, 16),
    ("f32", 8, 2, 64, 8),
    ("f16", 8, 2, 128, 16),
    ("f16", 8, 2, 64, 8),
    ("bf16", 12, 4, 96, 16),
    ("bf16", 8, 2, 128, 4),
    ("f16", 8, 2, 96, 8),
    ("f32", 8, 2, 96, 16),
    ("bf16", 16, 8, 256, 16),   # head_dim 256: the merge stores 1 KB rows, 16 bytes a lane
    ("f16", 8, 2, 256, 8),
    ("bf16", 32, 1, 128, 16),   # G = 32: one wavefront, two column groups
    ("f16", 33, 1, 64, 16),     # G = 33: two virtual heads; the row is stored once per KV head
    ("f16", 40, 2, 64, 8),      # G = 20
    ("f32", 34, 2, 64, 16),     # G = 17: 8 + 9
    ("bf16", 71, 1, 64, 16),    # G = 71: five virtual heads
    ("bf16", 36, 2, 64, 2),     # generic, G = 18
]


@pytest.mark.parametrize("dtype,Hq,Hkv,D,BS", SHAPES)
def test_fused_position_cases(dtype, Hq, Hkv, D, BS, split):
    """Last token, mid-context overwrite, first token, no token, and a
    position past T_b (written, not attended), against the oracle and
    bit-identical to the two-call form."""
    say(f"fused positions {dtype} Hq={Hq} Hkv={Hkv} D={D} BS={BS}")
    lens = [1, BS, BS + 1, 33, 100, 257, 64, 5, 0, 40, 0]
    positions = [0, BS - 1, BS, 17, -1, 256, 70, 2, -3, 0, 5]
    w = custom(dtype, len(lens), Hq, Hkv, D, BS, lens, positions, L=2, layer=1)
    # 70 >= T = 64 and the last, empty sequence's 5: written, never attended;
    # the other empty sequence's -3: skipped
    poison_append_slots(w, positions)
    two = DeviceWorkload(w)
    fused = DeviceWorkload(w)
    out = run_fused(fused, positions)
    ref_pool, ref = oracle_step(w, positions)
    assert_attention_close(out, ref, dtype, what="fused positions",
                           vmax=workload_vmax(w, pool=ref_pool))
    assert dev_to_np(fused.pool.data).tobytes() == ref_pool.tobytes()
    pos = torch.from_numpy(np.asarray(positions, np.int32)).cuda()
    pk.kv_append(two.pool, w.layer, two.k_new, two.v_new, two.tables, pos)
    out2 = two.decode()
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16) if out.element_size() == 2 else out,
                       out2.view(torch.int16) if out2.element_size() == 2 else out2), \
        "fused output differs from append + decode"
    assert not dev_to_np(out)[[8, 10]].any(), "empty sequences must give zero rows"


@pytest.mark.parametrize("idx", [2, 3, 4])
def test_fused_step_full_size(idx):
    """The benchmarked configurations (the Llama-shaped layer, the long
    contexts, the high-concurrency batch) at full size, through the
    benchmarked call: every output row against the oracle, the whole pool
    bit-exact against the oracle's append."""
    say(f"fused append+decode workload {idx} full size, every row")
    w = make_workload(idx)
    positions = w.positions.copy()
    poison_append_slots(w, positions)
    dw = DeviceWorkload(w)
    out = run_fused(dw, positions)
    ref_pool = oracle.kv_append(w.pool, w.layer, w.block_tables, positions, w.k_new, w.v_new)
    ref = oracle.paged_attention_decode(ref_pool, w.dtype, w.layer, w.block_tables,
                                        w.context_lens, w.q, w.scale)
    assert_attention_close(out, ref, w.dtype, what=f"fused w{idx} full")
    assert dev_to_np(dw.pool.data).tobytes() == ref_pool.tobytes()
    # a second step over the same inputs reads the appended rows from the pool
    # (now holding the same values), so the output must not change
    out2 = torch.empty_like(out)
    pk.paged_attention_decode(out2, dw.q, dw.pool, w.layer, dw.tables, dw.lens, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))


def test_decode_plan_matches_direct_calls():
    """DecodePlan runs the same library calls on fixed tensors: bit-identical
    to the direct calls in deterministic settings (same kernels, same split)."""
    say("decode plan vs direct calls")
    w = make_workload(2, S=6)
    positions = w.positions.copy()
    a = DeviceWorkload(w)
    b = DeviceWorkload(w)
    out_a = torch.empty_like(a.q)
    out_b = torch.empty_like(b.q)
    pos_a = torch.from_numpy(positions).cuda()
    pos_b = torch.from_numpy(positions).cuda()
    plan = pk.DecodePlan(out_a, a.q, a.pool, w.layer, a.tables, a.lens, w.scale,
                         a.k_new, a.v_new, pos_a)
    plan.run()
    pk.paged_attention_decode_append(out_b, b.q, b.pool, w.layer, b.tables, b.lens, w.scale,
                                     b.k_new, b.v_new, pos_b)
    torch.cuda.synchronize()
    assert dev_to_np(out_a).tobytes() == dev_to_np(out_b).tobytes()
    assert dev_to_np(a.pool.data).tobytes() == dev_to_np(b.pool.data).tobytes()
    plain = pk.DecodePlan(out_a, a.q, a.pool, w.layer, a.tables, a.lens, w.scale)
    plain.run()
    pk.paged_attention_decode(out_b, b.q, b.pool, w.layer, b.tables, b.lens, w.scale)
    torch.cuda.synchronize()
    assert dev_to_np(out_a).tobytes() == dev_to_np(out_b).tobytes()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        with pytest.raises(RuntimeError):
            plain.run()
