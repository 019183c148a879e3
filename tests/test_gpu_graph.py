"""The decode step captured in a HIP graph (torch.cuda.CUDAGraph around a
DecodePlan with its own workspace): every replay, with eager work and
synchronisations between replays, gives the eager result bit for bit, for
the plain decode and for the fused append + decode, and a replay after the
inputs were updated in place matches an eager call on the same inputs.  The
library records no memset and allocates nothing, so a capture holds only
its two kernels per call."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import paged_kv_cache_resolve_amd as pk
from workloads import make_workload

from gpu_helpers import DeviceWorkload, np_to_dev, say

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU"),
]


def bits(t: torch.Tensor) -> bytes:
    t = t.detach().contiguous()
    if t.element_size() == 2:
        t = t.view(torch.int16)
    return t.cpu().numpy().tobytes()


def capture(fn):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()                                   # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("fused,idx,S", [(False, 2, 6), (True, 2, 6), (True, 0, None),
                                         (False, 0, None), (True, 1, None), (True, 6, 4)])
def test_graph_replays_match_eager(fused, idx, S, split):
    say(f"graph replay fused={fused} workload {idx} S={S}")
    w = make_workload(idx, **({"S": S} if S else {}))
    dw = DeviceWorkload(w)
    out = torch.empty_like(dw.q)
    ws = torch.empty(pk.paged_attention_workspace_bytes(dw.pool, w.S, w.Hq), dtype=torch.uint8,
                     device="cuda")
    extra = (dw.k_new, dw.v_new, dw.positions) if fused else ()
    plan = pk.DecodePlan(out, dw.q, dw.pool, w.layer, dw.tables, dw.lens, w.scale, *extra,
                         workspace=ws)
    plan.run()
    torch.cuda.synchronize()
    want_out, want_pool = bits(out), bits(dw.pool.data)

    g = capture(plan.run)
    for i in range(4):
        out.fill_(float("nan"))                # eager work between replays
        ws.fill_(0xAB)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert bits(out) == want_out, f"replay {i} differs from the eager call"
        assert bits(dw.pool.data) == want_pool, f"replay {i} changed the pool differently"

    # new inputs written in place, then a replay against an eager call on the same inputs
    rng = np.random.default_rng(idx)
    q2 = rng.standard_normal(tuple(dw.q.shape), dtype=np.float32)
    if w.dtype == "bf16":
        from workloads import bf16_round_bits
        q2 = bf16_round_bits(q2)
    elif w.dtype == "f16":
        q2 = q2.astype(np.float16)
    dw.q.copy_(np_to_dev(q2, w.dtype))
    g.replay()
    torch.cuda.synchronize()
    replayed = bits(out)
    out.fill_(float("nan"))
    plan.run()
    torch.cuda.synchronize()
    assert replayed == bits(out)
