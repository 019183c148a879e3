"""GPU parity of the two multi-row appends, bit-exact over the whole pool:

- kv_append_layers (one token per sequence, every layer in one launch)
  against the oracle's all-layer append, and against one kv_append per layer;
- kv_append_tokens (several consecutive tokens per sequence: a prompt, or a
  chunk continuing a sequence) against the oracle's multi-token append.

The pool background is random bits, so a write to a wrong slot, layer or
head, or a missing write, changes bytes the comparison sees.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_resolve_amd as pk
from workloads import bf16_round_bits, make_append_batch

from gpu_helpers import assert_attention_close, dev_to_np, np_to_dev, say, t_dtype

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU"),
]

# dtype, Hkv, D, BS, L
SHAPES = [
    ("bf16", 8, 128, 16, 4),
    ("bf16", 2, 64, 16, 3),
    ("bf16", 1, 128, 32, 2),
    ("bf16", 2, 64, 8, 2),
    ("bf16", 4, 256, 16, 2),
    ("f32", 4, 64, 16, 3),
    ("f32", 2, 32, 8, 2),
    ("bf16", 3, 96, 16, 2),     # 12 units per head row, 3 heads: no power of two
    ("f32", 5, 20, 8, 2),       # 5 units per head row
    ("f16", 8, 128, 16, 3),
    ("f16", 2, 64, 32, 2),
]

# Ragged counts: empty, single token, a whole block, block + 1, many blocks;
# starts at 0 (a prompt), mid-block (a chunk continuing a sequence), on a block
# boundary ("BS" below), and negative (skipped although it has rows).
STARTS = [0, 0, 5, "BS", -1, 0, 37, 0, 3]
COUNTS = [1, 16, 11, 17, 4, 0, 70, 100, 1]


class DevicePool:
    def __init__(self, a):
        self.a = a
        data = np_to_dev(a.pool, a.dtype)
        self.pool = pk.KVPool(a.NB, a.BS, a.L, a.Hkv, a.D, t_dtype(a.dtype), data=data)
        self.tables = torch.from_numpy(a.block_tables).cuda()

    def pool_bytes(self) -> bytes:
        return dev_to_np(self.pool.data).tobytes()


def batch_for(dtype, Hkv, D, BS, L, seed=11, starts=STARTS, counts=COUNTS):
    st = [BS if s == "BS" else s for s in starts]
    return make_append_batch(seed, dtype=dtype, Hkv=Hkv, D=D, BS=BS, L=L, layer=L - 1,
                             starts=st, counts=counts)


@pytest.mark.parametrize("dtype,Hkv,D,BS,L", SHAPES)
def test_append_layers_matches_oracle(dtype, Hkv, D, BS, L):
    say(f"kv_append_layers {dtype} Hkv={Hkv} D={D} BS={BS} L={L}")
    a = batch_for(dtype, Hkv, D, BS, L)
    dp = DevicePool(a)
    pos = torch.from_numpy(a.start_positions).cuda()
    pk.kv_append_layers(dp.pool, np_to_dev(a.k_layers, dtype), np_to_dev(a.v_layers, dtype),
                        dp.tables, pos)
    torch.cuda.synchronize()
    ref = oracle.kv_append_layers(a.pool, a.block_tables, a.start_positions, a.k_layers,
                                  a.v_layers)
    assert dp.pool_bytes() == ref.tobytes(), "pool differs from the oracle's all-layer append"
    # and the same bytes as one single-layer append per layer
    single = DevicePool(a)
    for layer in range(L):
        k = np_to_dev(np.ascontiguousarray(a.k_layers[:, layer]), dtype)
        v = np_to_dev(np.ascontiguousarray(a.v_layers[:, layer]), dtype)
        pk.kv_append(single.pool, layer, k, v, single.tables, pos)
    torch.cuda.synchronize()
    assert single.pool_bytes() == dp.pool_bytes()


@pytest.mark.parametrize("dtype,Hkv,D,BS,L", SHAPES)
def test_append_tokens_matches_oracle(dtype, Hkv, D, BS, L):
    say(f"kv_append_tokens {dtype} Hkv={Hkv} D={D} BS={BS} L={L}")
    a = batch_for(dtype, Hkv, D, BS, L)
    dp = DevicePool(a)
    pk.kv_append_tokens(dp.pool, a.layer, np_to_dev(a.k_rows, dtype), np_to_dev(a.v_rows, dtype),
                        dp.tables, torch.from_numpy(a.start_positions).cuda(),
                        torch.from_numpy(a.token_offsets).cuda())
    torch.cuda.synchronize()
    ref = oracle.kv_append_tokens(a.pool, a.layer, a.block_tables, a.start_positions,
                                  a.token_offsets, a.k_rows, a.v_rows)
    assert dp.pool_bytes() == ref.tobytes(), "pool differs from the oracle's multi-token append"


def test_append_tokens_then_decode_sees_prompt():
    """A prompt written by kv_append_tokens is what decode attends over: the
    decode output equals the oracle's over the oracle-appended pool."""
    say("kv_append_tokens then decode")
    counts = [1, 16, 17, 40, 129, 3]
    a = make_append_batch(21, dtype="bf16", Hkv=2, D=128, BS=16, L=2, layer=1,
                          starts=[0] * len(counts), counts=counts)
    # a finite pool: the decode reads only appended rows, but keep NaN bits out anyway
    a.pool[...] = 0
    dp = DevicePool(a)
    pk.kv_append_tokens(dp.pool, a.layer, np_to_dev(a.k_rows, "bf16"),
                        np_to_dev(a.v_rows, "bf16"), dp.tables,
                        torch.from_numpy(a.start_positions).cuda(),
                        torch.from_numpy(a.token_offsets).cuda())
    ref_pool = oracle.kv_append_tokens(a.pool, a.layer, a.block_tables, a.start_positions,
                                       a.token_offsets, a.k_rows, a.v_rows)
    lens = np.asarray(counts, dtype=np.int32)
    rng = np.random.default_rng(5)
    q = bf16_round_bits(rng.standard_normal((len(counts), 8, 128), dtype=np.float32))
    out = torch.empty((len(counts), 8, 128), dtype=torch.bfloat16, device="cuda")
    scale = 128 ** -0.5
    pk.paged_attention_decode(out, np_to_dev(q, "bf16"), dp.pool, a.layer, dp.tables,
                              torch.from_numpy(lens).cuda(), scale)
    torch.cuda.synchronize()
    ref = oracle.paged_attention_decode(ref_pool, "bf16", a.layer, a.block_tables, lens, q, scale)
    assert_attention_close(out, ref, "bf16", what="decode after prompt append")


def test_append_tokens_prompt_llama8b_shape():
    """64 prompts of 512 tokens each (32768 rows), Llama-8B KV geometry
    (8 KV heads, head_dim 128, block 16, bf16) in a 4-layer pool; the whole
    pool bit-exact against the oracle."""
    say("kv_append_tokens 64 x 512 prompt, Llama-8B KV geometry")
    S = 64
    a = make_append_batch(31, dtype="bf16", Hkv=8, D=128, BS=16, L=4, layer=2,
                          starts=[0] * S, counts=[512] * S)
    dp = DevicePool(a)
    pk.kv_append_tokens(dp.pool, a.layer, np_to_dev(a.k_rows, "bf16"),
                        np_to_dev(a.v_rows, "bf16"), dp.tables,
                        torch.from_numpy(a.start_positions).cuda(),
                        torch.from_numpy(a.token_offsets).cuda())
    torch.cuda.synchronize()
    oracle.kv_append_tokens(a.pool, a.layer, a.block_tables, a.start_positions,
                            a.token_offsets, a.k_rows, a.v_rows, in_place=True)
    assert dp.pool_bytes() == a.pool.tobytes()


@pytest.mark.parametrize("tokens", [64, 160])
def test_append_tokens_mid_sizes(tokens):
    """Launch sizes between the small cases and the 64 x 512 prompt, so that
    every units-per-thread variant of the append kernel runs."""
    say(f"kv_append_tokens 64 x {tokens}, Llama-8B KV geometry")
    S = 64
    rng = np.random.default_rng(tokens)
    starts = rng.integers(0, 40, size=S)
    a = make_append_batch(51 + tokens, dtype="bf16", Hkv=8, D=128, BS=16, L=2, layer=1,
                          starts=starts, counts=rng.integers(tokens // 2, 2 * tokens, size=S))
    dp = DevicePool(a)
    pk.kv_append_tokens(dp.pool, a.layer, np_to_dev(a.k_rows, "bf16"),
                        np_to_dev(a.v_rows, "bf16"), dp.tables,
                        torch.from_numpy(a.start_positions).cuda(),
                        torch.from_numpy(a.token_offsets).cuda())
    torch.cuda.synchronize()
    oracle.kv_append_tokens(a.pool, a.layer, a.block_tables, a.start_positions,
                            a.token_offsets, a.k_rows, a.v_rows, in_place=True)
    assert dp.pool_bytes() == a.pool.tobytes()


def test_append_layers_llama8b_shape():
    """One decode token for 64 sequences in every layer of a 32-layer pool
    (Llama-8B KV geometry); every layer bit-exact against the oracle."""
    say("kv_append_layers 64 sequences x 32 layers")
    S = 64
    rng = np.random.default_rng(41)
    starts = rng.integers(0, 200, size=S)
    a = make_append_batch(41, dtype="bf16", Hkv=8, D=128, BS=16, L=32, layer=0,
                          starts=starts, counts=[1] * S, spare_blocks=0)
    dp = DevicePool(a)
    pk.kv_append_layers(dp.pool, np_to_dev(a.k_layers, "bf16"), np_to_dev(a.v_layers, "bf16"),
                        dp.tables, torch.from_numpy(a.start_positions).cuda())
    torch.cuda.synchronize()
    oracle.kv_append_layers(a.pool, a.block_tables, a.start_positions, a.k_layers, a.v_layers,
                            in_place=True)
    assert dp.pool_bytes() == a.pool.tobytes()
