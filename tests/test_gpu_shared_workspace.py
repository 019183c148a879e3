"""One decode workspace serving calls of different shapes in turn (as the
binding's per-stream workspace does): every call, plain or fused, under
both splits, matches the oracle whatever the previous call left in the
workspace; and calls alternating between two batches in one workspace give
the same bits every time (a merge that read a previous call's partials
would change them)."""

from __future__ import annotations

import pytest
import torch

import oracle
import paged_kv_cache_resolve_amd as pk
from workloads import make_workload

from gpu_helpers import DeviceWorkload, assert_attention_close, dev_to_np, say, workload_vmax

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU"),
]


def bits(t: torch.Tensor) -> bytes:
    return dev_to_np(t).tobytes()


def shared_workspace(dws):
    n = max(pk.paged_attention_workspace_bytes(d.pool, d.w.S, d.w.Hq) for d in dws)
    return torch.full((n,), 0x5A, dtype=torch.uint8, device="cuda")   # contents do not matter


@pytest.mark.parametrize("split", ["chunks", "auto"])
def test_one_workspace_across_shapes(split):
    say(f"shared workspace across shapes, split={split}")
    cases = [make_workload(2), make_workload(1), make_workload(4, S=40, seed_offset=2),
             make_workload(2, S=6, seed_offset=1), make_workload(0), make_workload(6, S=10)]
    dws = [DeviceWorkload(w) for w in cases]
    ws = shared_workspace(dws)
    for rnd in range(2):
        for i, d in enumerate(dws):
            w = d.w
            out = torch.empty_like(d.q)
            if rnd == 0:
                pk.paged_attention_decode(out, d.q, d.pool, w.layer, d.tables, d.lens, w.scale,
                                          workspace=ws, split=split)
            else:
                pk.paged_attention_decode_append(out, d.q, d.pool, w.layer, d.tables, d.lens,
                                                 w.scale, d.k_new, d.v_new, d.positions,
                                                 workspace=ws, split=split)
            torch.cuda.synchronize()
            ref_pool = w.pool if rnd == 0 else oracle.kv_append(
                w.pool, w.layer, w.block_tables, w.positions, w.k_new, w.v_new)
            ref = oracle.paged_attention_decode(ref_pool, w.dtype, w.layer, w.block_tables,
                                                w.context_lens, w.q, w.scale)
            assert_attention_close(out, ref, w.dtype, what=f"case {i} round {rnd}",
                                   vmax=workload_vmax(w, pool=ref_pool))


def test_alternating_batches_give_the_same_bits():
    say("alternating Llama-shaped and long-context batches in one workspace")
    a = DeviceWorkload(make_workload(2))
    b = DeviceWorkload(make_workload(3))
    ws = shared_workspace([a, b])
    outs = [torch.empty_like(a.q), torch.empty_like(b.q)]

    def run(i):
        d = (a, b)[i]
        pk.paged_attention_decode(outs[i], d.q, d.pool, d.w.layer, d.tables, d.lens, d.w.scale,
                                  workspace=ws, split="chunks")

    run(0)
    run(1)
    torch.cuda.synchronize()
    want = [bits(outs[0]), bits(outs[1])]
    for i, d in enumerate((a, b)):
        w = d.w
        ref = oracle.paged_attention_decode(w.pool, w.dtype, w.layer, w.block_tables,
                                            w.context_lens, w.q, w.scale)
        assert_attention_close(outs[i], ref, w.dtype, what=f"batch {i}")
    for rep in range(12):
        for i in (0, 1):
            outs[i].fill_(float("nan"))
        run(0)
        run(1)
        run(0)
        torch.cuda.synchronize()
        assert bits(outs[0]) == want[0], f"repeat {rep}: Llama-shaped batch changed"
        assert bits(outs[1]) == want[1], f"repeat {rep}: long-context batch changed"
