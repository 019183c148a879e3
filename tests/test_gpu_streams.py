"""Two decode steps in flight at once on two streams (default priority),
each with its own pool and workspace: the library keeps no device state of
its own, so each result equals the same step run alone."""

from __future__ import annotations

import pytest
import torch

import paged_kv_cache_resolve_amd as pk
from workloads import make_workload

from gpu_helpers import DeviceWorkload, say

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU"),
]


def bits(t):
    t = t.detach().contiguous()
    return (t.view(torch.int16) if t.element_size() == 2 else t).cpu().numpy().tobytes()


def test_two_streams_concurrently():
    say("two streams")
    wa = make_workload(2, S=24)
    wb = make_workload(4, S=40, seed_offset=1)
    a, b = DeviceWorkload(wa), DeviceWorkload(wb)
    plans, outs = [], []
    for dw, w in ((a, wa), (b, wb)):
        out = torch.empty_like(dw.q)
        outs.append(out)
        ws = torch.empty(pk.paged_attention_workspace_bytes(dw.pool, w.S, w.Hq),
                         dtype=torch.uint8, device="cuda")
        plans.append(pk.DecodePlan(out, dw.q, dw.pool, w.layer, dw.tables, dw.lens, w.scale,
                                   dw.k_new, dw.v_new, dw.positions, workspace=ws))
    # alone, one after the other
    plans[0].run()
    plans[1].run()
    torch.cuda.synchronize()
    alone = [bits(o) for o in outs]
    pools = [bits(a.pool.data), bits(b.pool.data)]
    # together, interleaved on two streams, several times
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for _ in range(5):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        with torch.cuda.stream(s1):
            plans[0].run()
        with torch.cuda.stream(s2):
            plans[1].run()
        with torch.cuda.stream(s1):
            plans[0].run()
        torch.cuda.synchronize()
        assert [bits(o) for o in outs] == alone
        assert [bits(a.pool.data), bits(b.pool.data)] == pools
