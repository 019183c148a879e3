"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.  Resolve, gather and append must match bit for bit;
attention must match within max-abs 1e-4 (fp32) or 2e-2 + 2e-2|ref| (bf16).
"""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_resolve_amd as pk
from paged_kv_cache_resolve_amd import _lib
from workloads import make_workload

from gpu_helpers import (NAN_BITS, DeviceWorkload, assert_attention_close, dev_to_np, np_to_dev, say,
                         workload_vmax,
                         t_dtype)

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU"),
]



def poison(w):
    """NaN into every pool slot no sequence owns (all layers, K and V) and
    garbage into unused table entries; returns the workload, modified."""
    slots = oracle.resolve_slots(w.block_tables, w.context_lens, w.BS, max(w.max_len, 1))
    used = np.zeros(w.NB * w.BS, dtype=bool)
    used[slots[slots >= 0]] = True
    used = used.reshape(w.NB, w.BS)
    blk, off = np.nonzero(~used)
    w.pool[blk, :, :, :, off, :] = NAN_BITS[w.dtype]
    w.block_tables = np.where(w.block_tables < 0, np.int32(2**31 - 1), w.block_tables).astype(np.int32)
    return w


def custom(dtype, S, Hq, Hkv, D, BS, lens, L=1, layer=0, seed_offset=0, nb_slack=3):
    lens = np.asarray(lens, dtype=np.int32)
    mb = max(1, max(math.ceil(int(t) / BS) for t in lens))
    nb = sum(math.ceil(int(t) / BS) for t in lens) + nb_slack
    return make_workload(0, dtype=dtype, S=S, Hq=Hq, Hkv=Hkv, D=D, BS=BS, L=L, layer=layer,
                         context_lens=lens, MB=mb, NB=nb, tables="perm", seed_offset=seed_offset)


# ----------------------------------------------------------------------------
# resolve
# ----------------------------------------------------------------------------

def test_resolve_page_examples():
    say("resolve page examples")
    tables = torch.tensor([[14, 89, 3], [4, 1, 7]], dtype=torch.int32, device="cuda")
    lens = torch.tensor([41, 41], dtype=torch.int32, device="cuda")
    got = pk.paged_kv_resolve(tables, lens, 16, 48).cpu().numpy()
    ref = oracle.resolve_slots(tables.cpu().numpy(), lens.cpu().numpy(), 16, 48)
    assert got.tobytes() == ref.tobytes()
    assert got[0, 16] == 1424 and got[1, 40] == 120 and got[0, 41] == -1


@pytest.mark.parametrize("idx", [0, 1, 4])
def test_resolve_workloads(idx):
    say(f"resolve workload {idx}")
    w = make_workload(idx, with_pool=False)
    max_len = w.max_len + 7
    tables = torch.from_numpy(w.block_tables).cuda()
    lens = torch.from_numpy(w.context_lens).cuda()
    got = pk.paged_kv_resolve(tables, lens, w.BS, max_len).cpu().numpy()
    ref = oracle.resolve_slots(w.block_tables, w.context_lens, w.BS, max_len)
    assert got.tobytes() == ref.tobytes()


# ----------------------------------------------------------------------------
# gather
# ----------------------------------------------------------------------------

def _check_gather(w, max_len=None, rows=None):
    dw = DeviceWorkload(w)
    max_len = w.max_len if max_len is None else max_len
    k, v, mask = pk.paged_kv_gather(dw.pool, w.layer, dw.tables, dw.lens, max_len)
    rows = list(range(w.S)) if rows is None else rows
    sub = lambda a: a[rows]  # noqa: E731
    rk, rv, rm = oracle.paged_kv_gather(w.pool, w.layer, w.block_tables[rows], w.context_lens[rows],
                                        max_len)
    idx = torch.tensor(rows, device="cuda")
    assert dev_to_np(k.index_select(0, idx)).tobytes() == rk.tobytes()
    assert dev_to_np(v.index_select(0, idx)).tobytes() == rv.tobytes()
    assert sub(mask.cpu().numpy()).tobytes() == rm.tobytes()


@pytest.mark.parametrize("idx", [0, 1])
def test_gather_workloads(idx):
    say(f"gather workload {idx}")
    _check_gather(poison(make_workload(idx)), )


@pytest.mark.parametrize("dtype,D,BS", [("bf16", 128, 16), ("bf16", 64, 32), ("f32", 64, 16),
                                        ("bf16", 32, 8), ("f32", 128, 1), ("f16", 128, 16),
                                        ("f16", 64, 4)])
def test_gather_shapes_and_padding(dtype, D, BS):
    say(f"gather {dtype} D={D} BS={BS}")
    w = poison(custom(dtype, 6, 4, 2, D, BS, [0, 1, BS - 1 if BS > 1 else 1, BS, BS + 1, 3 * BS + 5],
                      L=2, layer=1))
    _check_gather(w, max_len=w.max_len + 3)


# ----------------------------------------------------------------------------
# append
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("idx,dtype", [(0, None), (1, None), (1, "f16"), (2, "f16")])
def test_append_whole_pool(idx, dtype):
    say(f"append workload {idx} {dtype or ''}")
    over = {"dtype": dtype} if dtype else {}
    if idx == 2:
        over["S"] = 8
    w = make_workload(idx, **over)
    dw = DeviceWorkload(w)
    pk.kv_append(dw.pool, w.layer, dw.k_new, dw.v_new, dw.tables, dw.positions)
    ref = oracle.kv_append(w.pool, w.layer, w.block_tables, w.positions, w.k_new, w.v_new)
    assert dev_to_np(dw.pool.data).tobytes() == ref.tobytes()


def test_append_skips_negative_positions():
    say("append negative positions")
    w = custom("bf16", 4, 4, 2, 64, 16, [5, 17, 1, 40], L=3, layer=2)
    dw = DeviceWorkload(w)
    pos = np.array([4, -1, 0, -7], np.int32)
    pk.kv_append(dw.pool, w.layer, dw.k_new, dw.v_new, dw.tables, torch.from_numpy(pos).cuda())
    ref = oracle.kv_append(w.pool, w.layer, w.block_tables, pos, w.k_new, w.v_new)
    assert dev_to_np(dw.pool.data).tobytes() == ref.tobytes()


# ----------------------------------------------------------------------------
# decode
# ----------------------------------------------------------------------------

def _oracle_decode(w, seqs=None):
    return oracle.paged_attention_decode(w.pool, w.dtype, w.layer, w.block_tables, w.context_lens,
                                         w.q, w.scale, seqs=seqs)


def test_decode_tiny_fp32(split):
    say("decode workload 0 (fp32)")
    w = poison(make_workload(0))
    dw = DeviceWorkload(w)
    assert_attention_close(dw.decode(), _oracle_decode(w), w.dtype, what="w0")


def test_append_then_decode_churned_pool(split):
    """Workload 1: append the new token, then decode layer 11 over it."""
    say("append+decode workload 1")
    w = make_workload(1)
    dw = DeviceWorkload(w)
    pk.kv_append(dw.pool, w.layer, dw.k_new, dw.v_new, dw.tables, dw.positions)
    out = dw.decode()
    oracle.kv_append(w.pool, w.layer, w.block_tables, w.positions, w.k_new, w.v_new, in_place=True)
    assert_attention_close(out, _oracle_decode(w), w.dtype, what="w1")


@pytest.mark.parametrize("idx,S", [(2, 6), (3, 2), (4, 24), (7, 6), (8, 8), (9, 24)])
def test_decode_reduced_batches(idx, S, split):
    """Named shapes with fewer sequences, every output compared."""
    say(f"decode workload {idx} with S={S}")
    w = poison(make_workload(idx, S=S))
    dw = DeviceWorkload(w)
    assert_attention_close(dw.decode(), _oracle_decode(w), w.dtype, what=f"w{idx} S={S}")


@pytest.mark.parametrize("idx", [2, 3, 7, 9])
def test_decode_full_size_every_row(idx):
    """Full-size workloads in the configuration the benchmark times (the
    Llama-shaped layer, the long contexts, head_dim 256, MQA at batch 256):
    every sequence, head and dim against the oracle, and a second call
    bit-identical to the first."""
    say(f"decode workload {idx} full size, every row")
    w = make_workload(idx)
    dw = DeviceWorkload(w)
    out = dw.decode()
    assert_attention_close(out, _oracle_decode(w), w.dtype, what=f"w{idx} full",
                           vmax=workload_vmax(w))
    again = dw.decode()
    assert torch.equal(out.view(torch.int16), again.view(torch.int16)), "decode not deterministic"


@pytest.mark.parametrize("Hq,Hkv,D,dtype", [(16, 8, 256, "bf16"), (32, 1, 128, "bf16"),
                                           (71, 1, 64, "f16")])
def test_decode_full_size_other_heads(Hq, Hkv, D, dtype):
    """The Llama-shaped lengths (batch 64, log-normal contexts) with other head
    shapes at full size: head_dim 256 (Gemma-like), MQA with 32 query heads,
    and a 71-query-head MQA layer; every sequence against the oracle."""
    say(f"decode full size Hq={Hq} Hkv={Hkv} D={D} {dtype}, every row")
    w = make_workload(2, Hq=Hq, Hkv=Hkv, D=D, dtype=dtype)
    dw = DeviceWorkload(w)
    out = dw.decode()
    assert_attention_close(out, _oracle_decode(w), w.dtype, what=f"Hq={Hq} D={D} full",
                           vmax=workload_vmax(w))


def check_gather_every_row(w, k, v, mask, group=16):
    """The gather's outputs against the oracle's, bit for bit, on every
    sequence, in groups of `group` sequences.  Each group is compared with
    the oracle's gather up to the group's longest context on the host (so
    the oracle's arrays stay small); past it, every K/V element of the
    padded rows must be +0.0 bits and every mask byte 0 (the oracle's
    padding), checked on the device."""
    max_len = k.shape[1]
    lens = w.context_lens.astype(np.int64)
    mask_host = mask.cpu().numpy()
    for g0 in range(0, w.S, group):
        rows = list(range(g0, min(w.S, g0 + group)))
        top = int(lens[rows].max())
        rk, rv, rm = oracle.paged_kv_gather(w.pool, w.layer, w.block_tables[rows],
                                            w.context_lens[rows], top)
        sl = slice(g0, g0 + len(rows))
        assert dev_to_np(k[sl, :top]).tobytes() == rk.tobytes(), f"K of rows {rows}"
        assert dev_to_np(v[sl, :top]).tobytes() == rv.tobytes(), f"V of rows {rows}"
        assert mask_host[sl, :top].tobytes() == rm.tobytes(), f"mask of rows {rows}"
        if top < max_len:
            assert not mask_host[sl, top:].any(), f"mask padding of rows {rows}"
            for t in (k, v):
                tail = t[sl, top:].reshape(-1)
                bits = tail.view(torch.int16) if tail.element_size() == 2 else tail.view(torch.int32)
                assert int(torch.count_nonzero(bits).item()) == 0, f"padding of rows {rows}"


def test_high_concurrency_step_full_size():
    """Workload 4 at full size: append the new token into each tail block,
    decode, then gather.  Every sequence's decode output against the oracle,
    and the gather bit for bit on every row (16384-token rows, 17 GB of
    output, element offsets past 2^31)."""
    say("workload 4 append -> decode -> gather, every row")
    w = make_workload(4)
    dw = DeviceWorkload(w)
    pk.kv_append(dw.pool, w.layer, dw.k_new, dw.v_new, dw.tables, dw.positions)
    out = dw.decode()
    k, v, mask = pk.paged_kv_gather(dw.pool, w.layer, dw.tables, dw.lens, w.max_len)
    torch.cuda.synchronize()
    oracle.kv_append(w.pool, w.layer, w.block_tables, w.positions, w.k_new, w.v_new, in_place=True)
    assert_attention_close(out, _oracle_decode(w), w.dtype, what="w4")
    check_gather_every_row(w, k, v, mask)
    assert k.numel() > 2**31
    assert int(mask.sum().item()) == int(w.context_lens.astype(np.int64).sum())


# shapes that exercise both pass-1 kernels, tails, empty sequences and poison
EDGE_CASES = [
    # dtype, Hq, Hkv, D, BS
    ("bf16", 8, 2, 128, 16),    # MFMA, G = 4
    ("bf16", 14, 2, 64, 16),    # MFMA, G = 7
    ("bf16", 16, 1, 128, 32),   # MFMA, G = 16
    ("bf16", 4, 4, 128, 64),    # MFMA, G = 1
    ("bf16", 8, 2, 64, 8),      # MFMA bf16, 8-token blocks (per-lane block lookups)
    ("bf16", 8, 2, 128, 4),     # MFMA bf16, 4-token blocks
    ("bf16", 6, 2, 64, 2),      # generic bf16 (2-token blocks)
    ("f32", 6, 2, 36, 16),      # generic fp32, head_dim 36: merge lanes of 4 dims (not a multiple of 8)
    ("f32", 4, 2, 100, 16),     # generic fp32, head_dim 100
    ("f32", 8, 2, 20, 8),       # generic fp32, head_dim 20
    ("bf16", 6, 2, 96, 16),     # MFMA bf16, head_dim 96 (12-byte V rows)
    ("bf16", 16, 2, 96, 32),    # MFMA bf16, head_dim 96, G = 8
    ("bf16", 6, 2, 96, 8),      # MFMA bf16, head_dim 96, 8-token blocks
    ("f32", 4, 4, 64, 16),      # MFMA fp32, MHA
    ("f32", 32, 8, 128, 16),    # MFMA fp32, G = 4
    ("f32", 14, 2, 128, 32),    # MFMA fp32, G = 7
    ("f32", 8, 2, 64, 8),       # generic fp32 (block size 8)
    ("f32", 6, 2, 96, 16),      # generic fp32 (head_dim 96)
    ("f16", 8, 2, 128, 16),     # MFMA fp16, G = 4
    ("f16", 14, 2, 64, 32),     # MFMA fp16, G = 7
    ("f16", 16, 1, 128, 16),    # MFMA fp16, G = 16
    ("f16", 8, 2, 64, 8),       # MFMA fp16, 8-token blocks
    ("f16", 14, 2, 64, 4),      # MFMA fp16, 4-token blocks, G = 7
    ("f16", 6, 2, 96, 16),      # MFMA fp16, head_dim 96
    ("bf16", 8, 2, 64, 1),      # generic, one token per block
    ("bf16", 8, 2, 128, 128),   # MFMA, 128-token blocks
    ("bf16", 8, 2, 256, 16),    # MFMA bf16, head_dim 256 (one 16-token tile per step)
    ("f16", 16, 8, 256, 32),    # MFMA fp16, head_dim 256, G = 2
    ("bf16", 16, 1, 256, 8),    # MFMA bf16, head_dim 256, 8-token blocks, G = 16
    ("f16", 4, 4, 256, 4),      # MFMA fp16, head_dim 256, 4-token blocks, MHA
    ("bf16", 40, 2, 256, 16),   # head_dim 256, G = 20: two virtual heads
    ("f32", 4, 1, 256, 32),     # generic fp32, head_dim 256
    ("f32", 16, 1, 64, 64),     # MFMA fp32, G = 16
    # more than 16 query heads per KV head: up to 32 in one wavefront (two
    # MFMA column groups: 16-bit, head_dim 64/128, BS a multiple of 16), else
    # ceil(G/W) virtual heads of floor- or ceil(G/q) query heads
    ("bf16", 32, 1, 128, 16),   # MQA, G = 32: one wavefront, 16 + 16 columns
    ("bf16", 40, 2, 64, 16),    # G = 20: 16 + 4 columns
    ("bf16", 17, 1, 128, 16),   # G = 17: 16 + 1 columns
    ("f16", 48, 2, 64, 32),     # G = 24: 16 + 8 columns
    ("bf16", 33, 1, 128, 16),   # G = 33: virtual heads of 16 (second group empty) and 17
    ("bf16", 34, 2, 128, 8),    # G = 17 with 8-token blocks: virtual heads of 8 + 9
    ("bf16", 71, 1, 64, 16),    # G = 71: virtual heads of 23 + 24 + 24
    ("f16", 64, 1, 96, 16),     # G = 64, head_dim 96: four virtual heads of 16
    ("f16", 51, 1, 128, 32),    # G = 51: virtual heads of 25 + 26
    ("f32", 48, 2, 64, 16),     # MFMA fp32, G = 24: two of 12
    ("f32", 38, 2, 128, 16),    # MFMA fp32, G = 19: 9 + 10
    ("bf16", 36, 2, 64, 2),     # generic, G = 18: two of 9
    ("f32", 17, 1, 96, 16),     # generic fp32, G = 17: 8 + 9
]


@pytest.mark.parametrize("dtype,Hq,Hkv,D,BS", EDGE_CASES)
def test_decode_edge_lengths_with_poison(dtype, Hq, Hkv, D, BS, split):
    say(f"decode edges {dtype} Hq={Hq} Hkv={Hkv} D={D} BS={BS}")
    lens = [0, 1, BS - 1, BS, BS + 1, 15, 16, 17, 63, 64, 65, 1000, 4 * BS + 3, 0]
    w = poison(custom(dtype, len(lens), Hq, Hkv, D, BS, lens, L=2, layer=1))
    dw = DeviceWorkload(w)
    out = dw.decode()
    ref = _oracle_decode(w)
    assert_attention_close(out, ref, dtype, what="edges", vmax=workload_vmax(w))
    zero_rows = [i for i, t in enumerate(lens) if t == 0]
    assert not dev_to_np(out)[zero_rows].any(), "empty sequences must give zero rows"


@pytest.mark.parametrize("dtype,D,BS", [("bf16", 128, 16), ("f32", 64, 16), ("f16", 128, 16),
                                        ("bf16", 128, 8)])
def test_decode_block_permutation_invariance(dtype, D, BS, split):
    say(f"decode permutation invariance {dtype}")
    w = custom(dtype, 9, 8, 2, D, BS, [300, 1, 17, 0, 900, 64, 33, 2048, 5], nb_slack=40)
    dw = DeviceWorkload(w)
    a = dw.decode()
    perm = np.random.default_rng(3).permutation(w.NB)
    pool2 = np.empty_like(w.pool)
    pool2[perm] = w.pool
    w.pool = pool2
    w.block_tables = np.where(w.block_tables >= 0, perm[np.maximum(w.block_tables, 0)], -1).astype(np.int32)
    b = DeviceWorkload(w).decode()
    assert dev_to_np(a).tobytes() == dev_to_np(b).tobytes()


def test_decode_scale_zero_is_mean_of_v(split):
    say("decode scale 0")
    w = custom("bf16", 3, 8, 2, 128, 16, [37, 300, 1])
    w.scale = 0.0
    dw = DeviceWorkload(w)
    out = dw.decode()
    ref = _oracle_decode(w)
    assert_attention_close(out, ref, "bf16", what="scale0")


def test_decode_many_short_sequences(split):
    say("decode 5000 short sequences")
    rng = np.random.default_rng(8)
    lens = rng.integers(0, 41, size=5000)
    w = custom("bf16", 5000, 8, 2, 64, 16, lens)
    dw = DeviceWorkload(w)
    out = dw.decode()
    assert_attention_close(out, _oracle_decode(w), "bf16", what="many")


def test_decode_rejects_mismatched_dtype():
    say("decode dtype mismatch")
    w = custom("bf16", 2, 4, 2, 64, 16, [5, 9])
    dw = DeviceWorkload(w)
    with pytest.raises(ValueError):
        pk.paged_attention_decode(torch.empty(2, 4, 64, device="cuda"), dw.q.float(), dw.pool, 0,
                                  dw.tables, dw.lens, 0.125)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_output_dtype_rounding(dtype):
    """16-bit outputs are the fp32 result rounded to nearest even.  With one
    cached token the softmax weight is exactly 1, so the output must be the
    single V row, bit for bit (for fp16 also through the probability scale)."""
    say(f"decode {dtype} rounding")
    w = custom(dtype, 2, 4, 4, 64, 16, [1, 1])
    dw = DeviceWorkload(w)
    out = dev_to_np(dw.decode())
    # T = 1: the output is exactly the single V row (weight 1), so bits match
    for b in range(2):
        K, V = oracle.gather_sequence(w.pool, 0, w.block_tables[b], 1)
        assert out[b].tobytes() == np.ascontiguousarray(V[0]).tobytes()


def test_decode_largest_batch_and_one_past_it():
    """16384 sequences (the most whose chunk prefix fits in LDS) with short
    and empty contexts; one more is refused before any launch."""
    say("decode 16384 sequences")
    rng = np.random.default_rng(16384)
    lens = rng.integers(0, 40, size=16384)
    w = custom("bf16", 16384, 8, 2, 64, 16, lens)
    dw = DeviceWorkload(w)
    out = dw.decode()
    torch.cuda.synchronize()
    assert_attention_close(out, _oracle_decode(w), "bf16", what="16384")
    zero = [i for i in range(16384) if lens[i] == 0]
    assert not dev_to_np(out)[zero].any()
    q = torch.zeros(16385, 8, 64, dtype=torch.bfloat16, device="cuda")
    tables = torch.zeros(16385, 1, dtype=torch.int32, device="cuda")
    ctx = torch.zeros(16385, dtype=torch.int32, device="cuda")
    with pytest.raises(pk.PagedKVError) as e:
        pk.paged_attention_decode(torch.empty_like(q), q, dw.pool, 0, tables, ctx, 0.125)
    assert e.value.status == _lib.ERR_UNSUPPORTED


def _rne_16(x32: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to bf16 / fp16 bits, nearest even, written out
    with integer arithmetic (bf16) or numpy's IEEE conversion (fp16)."""
    if dtype == "f16":
        return x32.astype(np.float16).view(np.uint16)
    u = x32.view(np.uint32).astype(np.uint64)
    lower = u >> 16
    rest = u & 0xFFFF
    up = (rest > 0x8000) | ((rest == 0x8000) & (lower & 1 == 1))
    return (lower + up).astype(np.uint16)


@pytest.mark.parametrize("dtype,D,BS", [("bf16", 128, 16), ("bf16", 64, 8), ("f16", 128, 16),
                                        ("f16", 64, 8)])
def test_output_rounding_is_nearest_even(dtype, D, BS, split):
    """Two cached tokens with identical K rows get weights of exactly 1/2,
    so the fp32 result is the midpoint of their V values.  V pairs are
    neighbouring representable values, so every midpoint lies exactly
    halfway between two outputs: round-to-nearest-even and truncation give
    different bits, and the output must be the even one."""
    say(f"output rounding {dtype} D={D} BS={BS}")
    w = custom(dtype, 3, 8, 2, D, BS, [2, 2, 2])
    rng = np.random.default_rng(D + BS)
    for b in range(w.S):
        blk = w.block_tables[b, 0]
        for g in range(w.Hkv):
            w.pool[blk, 0, 0, g, 1, :] = w.pool[blk, 0, 0, g, 0, :]       # K1 = K0
            if dtype == "f16":
                lo = (rng.standard_normal(D) * 4).astype(np.float16)
                hi = np.nextafter(lo, np.float16(np.inf) * np.sign(lo + np.float16(1e-3)))
            else:
                bits = w.pool[blk, 1, 0, g, 0, :].astype(np.uint32)
                lo = bits.astype(np.uint16)
                hi = (bits + 1).astype(np.uint16)                          # next bf16 away from 0
            w.pool[blk, 1, 0, g, 0, :] = lo
            w.pool[blk, 1, 0, g, 1, :] = hi
    out = dev_to_np(DeviceWorkload(w).decode())
    G = 4
    for b in range(w.S):
        blk = w.block_tables[b, 0]
        for h in range(8):
            v0 = oracle.widen(w.pool[blk, 1, 0, h // G, 0, :], dtype)
            v1 = oracle.widen(w.pool[blk, 1, 0, h // G, 1, :], dtype)
            mid = ((v0 + v1) / 2).astype(np.float32)                     # exact in fp32
            assert (mid.astype(np.float64) == (v0 + v1) / 2).all()
            want = _rne_16(mid, dtype)
            got = out[b, h].view(np.uint16)
            assert got.tobytes() == want.tobytes(), (b, h)
