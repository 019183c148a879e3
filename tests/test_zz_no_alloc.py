"""paged_attention_decode_noalloc: the decode with the library's static
device scratch instead of a caller's workspace (for callers that cannot
allocate).  Called through the C ABI and compared with
paged_attention_decode on the same inputs: two calls in a row, the second
with a smaller batch, each bit-identical to the workspace form under the
same split and within tolerance of the oracle on every row."""

from __future__ import annotations

import ctypes

import pytest
import torch

import oracle
import paged_kv_cache_resolve_amd as pk
from paged_kv_cache_resolve_amd import _lib
from workloads import make_workload

from gpu_helpers import DeviceWorkload, assert_attention_close, dev_to_np, say, workload_vmax

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU"),
]


def decode_noalloc(dw, flags: int) -> torch.Tensor:
    w = dw.w
    out = torch.empty_like(dw.q)
    rc = pk.library().paged_attention_decode_noalloc(
        out.data_ptr(), dw.q.data_ptr(), dw.pool.handle, w.layer, dw.tables.data_ptr(),
        int(dw.tables.shape[1]), dw.lens.data_ptr(), w.S, w.Hq, ctypes.c_float(w.scale), flags,
        torch.cuda.current_stream().cuda_stream)
    assert rc == _lib.OK, pk.library().pagedkv_status_string(rc)
    return out


@pytest.mark.parametrize("flags", [0, _lib.DECODE_CHUNKS])
def test_noalloc_matches_workspace_decode_two_calls(flags):
    """First the full Llama-shaped batch (64 sequences, 18 MB of scratch),
    then a 6-sequence batch of the same shape, then the churned-pool batch
    (the LDS-staged per-pair stream, by default) and the tiny fp32 batch:
    each noalloc call against the workspace call and the oracle."""
    cases = [(2, {}), (2, {"S": 6, "seed_offset": 3}), (1, {}), (0, {})]
    for idx, over in cases:
        say(f"noalloc decode workload {idx} {over} flags={flags}")
        w = make_workload(idx, **over)
        dw = DeviceWorkload(w)
        got = decode_noalloc(dw, flags)
        want = torch.empty_like(dw.q)
        pk.paged_attention_decode(want, dw.q, dw.pool, w.layer, dw.tables, dw.lens, w.scale,
                                  split=flags)
        torch.cuda.synchronize()
        assert dev_to_np(got).tobytes() == dev_to_np(want).tobytes(), f"workload {idx} {over}"
        ref = oracle.paged_attention_decode(w.pool, w.dtype, w.layer, w.block_tables,
                                            w.context_lens, w.q, w.scale)
        assert_attention_close(got, ref, w.dtype, what=f"noalloc w{idx}", vmax=workload_vmax(w))


def test_noalloc_refuses_a_call_past_its_scratch():
    """A batch whose workspace exceeds 64 MiB is refused before any launch;
    the next call that fits still runs correctly."""
    say("noalloc oversized call")
    w = make_workload(2, S=4)
    dw = DeviceWorkload(w)
    big = 8000
    assert pk.paged_attention_workspace_bytes(dw.pool, big, w.Hq) > (64 << 20)
    q = torch.zeros(big, w.Hq, w.D, dtype=torch.bfloat16, device="cuda")
    out = torch.full_like(q, 3.0)
    tables = torch.zeros(big, 1, dtype=torch.int32, device="cuda")
    lens = torch.zeros(big, dtype=torch.int32, device="cuda")
    rc = pk.library().paged_attention_decode_noalloc(
        out.data_ptr(), q.data_ptr(), dw.pool.handle, 0, tables.data_ptr(), 1, lens.data_ptr(),
        big, w.Hq, ctypes.c_float(0.1), 0, torch.cuda.current_stream().cuda_stream)
    assert rc == _lib.ERR_SCRATCH
    torch.cuda.synchronize()
    assert bool((out == 3.0).all().item()), "a refused call must not write"
    got = decode_noalloc(dw, 0)
    torch.cuda.synchronize()
    ref = oracle.paged_attention_decode(w.pool, w.dtype, w.layer, w.block_tables, w.context_lens,
                                        w.q, w.scale)
    assert_attention_close(got, ref, w.dtype, what="noalloc after refusal")
