"""GPU parity of the gather-then-dense path ([mini-infer] v0.2.0): the
batched gather, then dense_attention_decode over the padded batch, against
the oracle's masked dense decode (and so against the paged decode, which the
oracle pins it to).  Masks that are not prefixes, fully masked sequences and
max_len values that end inside a chunk are covered."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_resolve_amd as pk
from workloads import make_workload

from gpu_helpers import (DeviceWorkload, assert_attention_close, dense_vmax, dev_to_np, np_to_dev,
                         say, workload_vmax)

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU"),
]


def dense(q, k, v, mask, scale):
    out = torch.empty_like(q)
    pk.dense_attention_decode(out, q, k, v, mask, scale)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("idx,S,dtype", [(2, 6, "bf16"), (2, 6, "f16"), (1, None, "bf16"),
                                         (4, 24, "bf16"), (7, 6, "bf16"), (8, 6, "f16")])
def test_gather_then_dense_matches_oracle(idx, S, dtype):
    say(f"gather then dense, workload {idx} S={S} {dtype}")
    over = {"dtype": dtype}
    if S:
        over["S"] = S
    w = make_workload(idx, **over)
    dw = DeviceWorkload(w)
    k, v, mask = pk.paged_kv_gather(dw.pool, w.layer, dw.tables, dw.lens)
    out = dense(dw.q, k, v, mask, w.scale)
    kn, vn, mn = dev_to_np(k), dev_to_np(v), mask.cpu().numpy()
    ref = oracle.dense_masked_decode(kn, vn, mn, w.q, w.dtype, w.scale)
    vmax = workload_vmax(w)
    assert_attention_close(out, ref, w.dtype, what="dense", vmax=vmax)
    # the paged decode of the same batch, within the same tolerance of the same values
    paged = dw.decode()
    torch.cuda.synchronize()
    assert_attention_close(paged, ref, w.dtype, what="paged", vmax=vmax)


@pytest.mark.parametrize("dtype,Hq,Hkv,D", [("bf16", 8, 2, 128), ("f16", 14, 2, 64),
                                            ("bf16", 16, 1, 128), ("f16", 4, 4, 128),
                                            ("bf16", 6, 2, 96), ("bf16", 32, 1, 128),
                                            ("f16", 40, 2, 64), ("bf16", 34, 2, 128),
                                            ("bf16", 16, 8, 256), ("f16", 8, 2, 256)])
@pytest.mark.parametrize("max_len", [1, 31, 33, 200, 1000])
def test_dense_random_masks(dtype, Hq, Hkv, D, max_len):
    say(f"dense masks {dtype} Hq={Hq} Hkv={Hkv} D={D} max_len={max_len}")
    rng = np.random.default_rng(max_len * 7 + D)
    S = 7
    npdt = np.float16 if dtype == "f16" else np.float32
    k = rng.standard_normal((S, max_len, Hkv, D), dtype=np.float32).astype(npdt)
    v = rng.standard_normal((S, max_len, Hkv, D), dtype=np.float32).astype(npdt)
    q = rng.standard_normal((S, Hq, D), dtype=np.float32).astype(npdt)
    if dtype == "bf16":
        from workloads import bf16_round_bits
        k, v, q = bf16_round_bits(k), bf16_round_bits(v), bf16_round_bits(q)
    mask = (rng.random((S, max_len)) < 0.6).astype(np.uint8)
    mask[0] = 0                        # nothing to attend: zero row
    mask[1] = 1                        # everything
    mask[2] = 0
    mask[2, -1] = 1                    # only the last token (inside the last chunk)
    mask[3, :max_len // 2] = 0         # a masked prefix: early chunks see nothing
    scale = D ** -0.5
    out = dense(np_to_dev(q, dtype), np_to_dev(k, dtype), np_to_dev(v, dtype),
                torch.from_numpy(mask).cuda(), scale)
    ref = oracle.dense_masked_decode(k, v, mask, q, dtype, scale)
    assert_attention_close(out, ref, dtype, what="dense masks", vmax=dense_vmax(v, mask, dtype, Hq))
    assert not dev_to_np(out)[0].astype(np.float32).any()


def test_dense_empty_batch_and_zero_length():
    say("dense zero sizes")
    q = torch.zeros(3, 8, 128, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(3, 0, 2, 128, dtype=torch.bfloat16, device="cuda")
    mask = torch.zeros(3, 0, dtype=torch.uint8, device="cuda")
    out = torch.full_like(q, 7.0)
    pk.dense_attention_decode(out, q, k, k, mask, 0.1)
    torch.cuda.synchronize()
    assert not out.float().any()


def test_gather_then_dense_full_size_llama8b():
    """The Llama-shaped batch at full size (max_len = the longest context):
    every row against the oracle."""
    say("gather then dense, workload 2 full size, every row")
    w = make_workload(2)
    dw = DeviceWorkload(w)
    k, v, mask = pk.paged_kv_gather(dw.pool, w.layer, dw.tables, dw.lens)
    out = dense(dw.q, k, v, mask, w.scale)
    ref = oracle.paged_attention_decode(w.pool, w.dtype, w.layer, w.block_tables, w.context_lens,
                                        w.q, w.scale)
    assert_attention_close(out, ref, w.dtype, what="dense full")
