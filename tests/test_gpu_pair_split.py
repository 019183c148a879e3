"""The per-pair decode split (one workgroup of 8 wavefronts per (sequence,
KV head) pair, which merges its own pieces; at head_dim 64 in 16 bits the
LDS-staged stream, whose pairs get two workgroups, each with half of V's
dims, while those fit on the device at once) against the oracle, next to
the persistent chunk split on the same inputs.

Which split ran is read off the workspace: the chunk split's pass 1 writes
the per-sequence chunk prefix at the start of the workspace, the per-pair
kernel never touches it.
"""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_resolve_amd as pk
from workloads import make_workload

from gpu_helpers import NAN_BITS, DeviceWorkload, assert_attention_close, dev_to_np, say, workload_vmax

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU"),
]

SENTINEL = 0xA5


def workload(dtype, Hq, Hkv, D, BS, lens, L=1, layer=0):
    lens = np.asarray(lens, dtype=np.int32)
    mb = max(1, max(math.ceil(int(t) / BS) for t in lens))
    nb = sum(math.ceil(int(t) / BS) for t in lens) + 3
    w = make_workload(0, dtype=dtype, S=len(lens), Hq=Hq, Hkv=Hkv, D=D, BS=BS, L=L, layer=layer,
                      context_lens=lens, MB=mb, NB=nb, tables="perm")
    # NaN in every slot no sequence owns: the per-pair kernel must mask as the
    # chunk split does
    slots = oracle.resolve_slots(w.block_tables, w.context_lens, w.BS, max(w.max_len, 1))
    used = np.zeros(w.NB * w.BS, dtype=bool)
    used[slots[slots >= 0]] = True
    blk, off = np.nonzero(~used.reshape(w.NB, w.BS))
    w.pool[blk, :, :, :, off, :] = NAN_BITS[w.dtype]
    return w


def decode_with(dw, mode):
    """Decode under `mode` with a fresh workspace whose chunk-prefix section
    (its first bytes) holds a sentinel and the rest zeros (as a new
    workspace must be); returns the output and whether the chunk prefix was
    written (the chunk split ran)."""
    batch, hq = dw.q.shape[0], dw.q.shape[1]
    n = pk.paged_attention_workspace_bytes(dw.pool, batch, hq)
    ws = torch.zeros((n,), dtype=torch.uint8, device="cuda")
    ws[: 4 * (batch + 1)] = SENTINEL
    out = torch.empty_like(dw.q)
    pk.paged_attention_decode(out, dw.q, dw.pool, dw.w.layer, dw.tables, dw.lens, dw.w.scale,
                              workspace=ws, split=mode)
    torch.cuda.synchronize()
    prefix_written = bool((ws[: 4 * (batch + 1)] != SENTINEL).any().item())
    return out, prefix_written


def reference(w):
    return oracle.paged_attention_decode(w.pool, w.dtype, w.layer, w.block_tables,
                                         w.context_lens, w.q, w.scale)


PAIR_KV_BYTES = 256 << 10       # per (sequence, KV head): 8 wavefronts x 32 KiB
PAIR_KV_BYTES_LDS = 512 << 10   # the LDS-staged stream: 4 wavefronts x 128 KiB


def pair_kv_bytes(dtype, D, BS):
    """K/V bytes per (sequence, KV head) up to which the per-pair kernel runs:
    more for the LDS-staged stream (head_dim 64, 16-bit, blocks of a multiple
    of 16 tokens)."""
    lds = dtype != "f32" and D == 64 and BS % 16 == 0
    return PAIR_KV_BYTES_LDS if lds else PAIR_KV_BYTES


def longest_pair_tokens(dtype, D, BS):
    """The longest table span (a whole number of blocks) the per-pair kernel takes."""
    e = 4 if dtype == "f32" else 2
    return pair_kv_bytes(dtype, D, BS) // (2 * D * e) // BS * BS


def pair_lens(dtype, D, BS):
    """Lengths giving 0 chunks, 1 chunk (one wavefront sees the pair whole),
    2..7 chunks (fewer pieces than wavefronts), 8 and more (uneven pieces,
    and with the LDS-staged stream more chunks per wavefront than it has
    slots) and the longest pair the per-pair kernel takes."""
    c = 16 if dtype == "f32" else 32   # tokens per chunk at head_dim <= 128
    top = longest_pair_tokens(dtype, D, BS)
    lens = [0, 1, c - 1, c, c + 1, 3 * c + 5, 7 * c, 8 * c, 8 * c + 1, 12 * c + 3, 16 * c,
            16 * c + 1, 26 * c - 3, top - 1, top]
    assert top >= 8 * c + 1
    return sorted(set(t for t in lens if t <= top))


CASES = [
    ("bf16", 32, 8, 128, 16),
    ("bf16", 14, 2, 64, 16),
    ("bf16", 16, 1, 128, 32),
    ("f16", 8, 2, 128, 16),
    ("f16", 16, 2, 64, 16),
    ("f16", 12, 4, 96, 16),
    ("bf16", 8, 2, 64, 8),     # 8-token blocks
    ("f16", 8, 2, 128, 4),     # 4-token blocks
    ("bf16", 24, 1, 64, 8),    # 24 query heads on one KV head: two virtual heads of 12
    ("f32", 4, 4, 64, 16),
    ("f32", 32, 8, 128, 16),
    ("f32", 24, 1, 64, 16),    # two virtual heads of 12
]


@pytest.mark.parametrize("dtype,Hq,Hkv,D,BS", CASES)
def test_pair_split_matches_oracle_and_chunk_split(dtype, Hq, Hkv, D, BS):
    say(f"pair split {dtype} Hq={Hq} Hkv={Hkv} D={D} BS={BS}")
    lens = pair_lens(dtype, D, BS)
    w = workload(dtype, Hq, Hkv, D, BS, lens, L=2, layer=1)
    dw = DeviceWorkload(w)
    ref = reference(w)
    out_p, wrote_p = decode_with(dw, pk.SPLIT_AUTO)
    out_c, wrote_c = decode_with(dw, pk.SPLIT_CHUNKS)
    assert not wrote_p, "small batch did not take the per-pair split"
    assert wrote_c, "SPLIT_CHUNKS did not take the chunk split"
    vmax = workload_vmax(w)
    assert_attention_close(out_p, ref, dtype, what="per-pair split", vmax=vmax)
    assert_attention_close(out_c, ref, dtype, what="chunk split", vmax=vmax)
    zero_rows = [i for i, t in enumerate(lens) if t == 0]
    assert not dev_to_np(out_p)[zero_rows].any(), "empty sequences must give zero rows"
    # deterministic: the same call twice gives the same bits
    out_p2, _ = decode_with(dw, pk.SPLIT_AUTO)
    assert torch.equal(out_p.view(torch.int16) if out_p.element_size() == 2 else out_p,
                       out_p2.view(torch.int16) if out_p2.element_size() == 2 else out_p2)


@pytest.mark.parametrize("dtype,D,BS,extra,expect_pairs", [
    ("bf16", 64, 16, 0, True),     # 2048 tokens: the limit (LDS-staged stream)
    ("bf16", 64, 16, 16, False),   # one block more
    ("f16", 64, 16, 0, True),
    ("f16", 64, 16, 16, False),
    ("bf16", 64, 8, 0, True),      # 8-token blocks
    ("bf16", 64, 8, 8, False),
    ("bf16", 128, 16, 0, True),    # 512 tokens
    ("bf16", 128, 16, 16, False),
    ("f32", 64, 16, 0, True),      # 512 tokens
    ("f32", 64, 16, 16, False),
])
def test_pair_split_length_limit(dtype, D, BS, extra, expect_pairs):
    """The choice follows max_blocks_per_seq * block_size, and both sides of
    the limit match the oracle."""
    longest = longest_pair_tokens(dtype, D, BS) + extra
    say(f"pair split limit {dtype} D={D} BS={BS} longest={longest}")
    w = workload(dtype, 8, 2, D, BS, [longest, 5, 300])
    dw = DeviceWorkload(w)
    out, wrote = decode_with(dw, pk.SPLIT_AUTO)
    assert wrote != expect_pairs
    assert_attention_close(out, reference(w), dtype, what=f"limit {longest}",
                           vmax=workload_vmax(w))


def test_pair_split_not_taken_for_many_pairs():
    """4096 (sequence, KV head) pairs: more workgroups than the GPU holds at
    once, so the chunk split runs."""
    say("pair split not taken: 512 sequences x 8 KV heads")
    rng = np.random.default_rng(5)
    lens = rng.integers(1, 200, size=512)
    w = workload("bf16", 32, 8, 128, 16, lens)
    dw = DeviceWorkload(w)
    out, wrote = decode_with(dw, pk.SPLIT_AUTO)
    assert wrote
    assert_attention_close(out, reference(w), "bf16", what="many pairs")


def test_pair_split_named_small_workloads():
    """By default the tiny fp32 batch and the churned-pool batch (tables of
    2048 tokens at head_dim 64, bf16: the LDS-staged stream) take the
    per-pair split."""
    for idx, expect_pairs in ((0, True), (1, True)):
        say(f"pair split named workload {idx}")
        w = make_workload(idx)
        dw = DeviceWorkload(w)
        out, wrote = decode_with(dw, pk.SPLIT_AUTO)
        assert wrote != expect_pairs, f"workload {idx}: unexpected split"
        assert_attention_close(out, reference(w), w.dtype, what=f"workload {idx}",
                               vmax=workload_vmax(w))


def _score_pattern_workload(dtype):
    """Four sequences on the LDS-staged per-pair stream (bf16/fp16, head_dim
    64, 16-token blocks, 7 query heads per KV head) whose scores follow set
    patterns: every query row is 1.0 in dim 0 and 0 elsewhere, and K's dim 0
    is chosen so that scale * q.k_t = s(t) for every head.  The patterns make
    the running max grow in every chunk (s = 0.01 t), never after the first
    (s = -0.01 t), jump by 15 (21.6 in log2 units, past the lazy-rescale
    threshold of 8) halfway, and grow by 4.5 in all (6.5 in log2 units, under
    the threshold), so that probabilities above 1 meet the stale reference."""
    from workloads import bf16_round_bits
    lens = [2048, 2048, 2048, 1500]
    w = workload(dtype, 14, 2, 64, 16, lens)
    patterns = [lambda t: 0.01 * t, lambda t: -0.01 * t,
                lambda t: np.where(t < 1024, 0.0, 15.0), lambda t: 0.003 * t]
    store = (lambda x: bf16_round_bits(np.asarray(x, np.float32))) if dtype == "bf16" else \
        (lambda x: np.asarray(x, np.float16))
    q = np.zeros((w.S, w.Hq, w.D), np.float32)
    q[:, :, 0] = 1.0
    w.q = store(q)
    for b, f in enumerate(patterns):
        t = np.arange(int(w.context_lens[b]))
        blks = w.block_tables[b, t // w.BS]
        offs = t % w.BS
        k0 = store(np.asarray(f(t), np.float32) / np.float32(w.scale))
        w.pool[blks, 0, w.layer, :, offs, 0] = k0[:, None]
    return w


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_lds_stream_running_max_patterns(dtype):
    """The LDS-staged stream's rescale taken only when a column's max grows
    past the threshold, and the normaliser summed by the MFMA unit, against
    the oracle and the chunk split on score patterns that force each path."""
    say(f"LDS stream running-max patterns {dtype}")
    w = _score_pattern_workload(dtype)
    dw = DeviceWorkload(w)
    ref = reference(w)
    out_p, wrote_p = decode_with(dw, pk.SPLIT_AUTO)
    out_c, wrote_c = decode_with(dw, pk.SPLIT_CHUNKS)
    assert not wrote_p and wrote_c
    vmax = workload_vmax(w)
    assert_attention_close(out_p, ref, dtype, what="per-pair, score patterns", vmax=vmax)
    assert_attention_close(out_c, ref, dtype, what="chunk split, score patterns", vmax=vmax)


def _random_pair_cases(n=24, seed=2024):
    """Seeded shapes for the LDS-staged per-pair stream: 16-bit, head_dim 64,
    block sizes that are multiples of 16 (48 and 80 among them, so a table
    entry is found by a true division), 1 to 16 query heads per KV head,
    lengths from 0 up to the 512 KiB per-pair limit."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        dtype = ["bf16", "f16"][i % 2]
        BS = int(rng.choice([16, 32, 48, 64, 80]))
        Hkv = int(rng.choice([1, 2, 4, 8]))
        G = int(rng.integers(1, 17))
        S = int(rng.integers(1, 24))
        top = (512 << 10) // (2 * 64 * 2) // BS * BS
        lens = rng.integers(0, top + 1, size=S)
        lens[rng.integers(0, S)] = int(rng.integers(top // 2, top + 1))   # one long pair
        cases.append((dtype, G * Hkv, Hkv, BS, [int(x) for x in lens]))
    return cases


@pytest.mark.parametrize("case", range(24))
def test_lds_stream_random_shapes(case):
    dtype, Hq, Hkv, BS, lens = _random_pair_cases()[case]
    say(f"LDS stream random case {case}: {dtype} Hq={Hq} Hkv={Hkv} BS={BS} S={len(lens)} "
        f"max T={max(lens)}")
    w = workload(dtype, Hq, Hkv, 64, BS, lens, L=2, layer=1)
    dw = DeviceWorkload(w)
    out, wrote = decode_with(dw, pk.SPLIT_AUTO)
    assert not wrote, "expected the per-pair split"
    assert_attention_close(out, reference(w), dtype, what=f"random case {case}",
                           vmax=workload_vmax(w))
    zero_rows = [i for i, t in enumerate(lens) if t == 0]
    assert not dev_to_np(out)[zero_rows].any(), "empty sequences must give zero rows"


@pytest.mark.parametrize("S", [64, 65])
def test_lds_stream_split_v_limit(S):
    """Two workgroups per pair (half of V's dims each) while twice the pair
    count, rounded up to a multiple of 8, fits on the 256 CUs: 64 sequences x
    2 KV heads (grid 256) take that form, 65 (grid 264) one workgroup per
    pair.  Both against the oracle."""
    say(f"LDS stream split-V limit: {S} sequences x 2 KV heads")
    rng = np.random.default_rng(1000 + S)
    lens = rng.integers(0, 700, size=S)
    lens[0] = 640
    w = workload("bf16", 14, 2, 64, 16, lens)
    dw = DeviceWorkload(w)
    out, wrote = decode_with(dw, pk.SPLIT_AUTO)
    assert not wrote, "expected the per-pair split"
    assert_attention_close(out, reference(w), "bf16", what=f"{S} sequences")


@pytest.mark.parametrize("S,Hkv", [(1, 1), (3, 1), (5, 3), (9, 1)])
def test_lds_stream_split_v_partial_grid(S, Hkv):
    """Pair counts that are not a multiple of 8: the split-V grid is rounded
    up, and the workgroups past the last pair exit at once.  Every output
    row (both halves of every head) against the oracle."""
    say(f"LDS stream split-V partial grid: S={S} Hkv={Hkv}")
    rng = np.random.default_rng(77 + 10 * S + Hkv)
    lens = rng.integers(1, 1200, size=S)
    w = workload("f16", 4 * Hkv, Hkv, 64, 32, lens, L=3, layer=2)
    dw = DeviceWorkload(w)
    out, wrote = decode_with(dw, pk.SPLIT_AUTO)
    assert not wrote, "expected the per-pair split"
    assert_attention_close(out, reference(w), "f16", what=f"S={S} Hkv={Hkv}",
                           vmax=workload_vmax(w))


@pytest.mark.parametrize("S,expect_pairs", [(128, True), (129, False)])
def test_lds_stream_resident_limit(S, expect_pairs):
    """The LDS-staged stream takes 128 KiB of LDS per workgroup, one per CU:
    256 (sequence, KV head) pairs fit on the 256 CUs at once, 258 do not and
    run on the chunk split; both against the oracle."""
    say(f"LDS stream resident limit: {S} sequences x 2 KV heads")
    rng = np.random.default_rng(S)
    lens = rng.integers(0, 300, size=S)
    w = workload("bf16", 14, 2, 64, 16, lens)
    dw = DeviceWorkload(w)
    out, wrote = decode_with(dw, pk.SPLIT_AUTO)
    assert wrote != expect_pairs
    assert_attention_close(out, reference(w), "bf16", what=f"{S} sequences")
