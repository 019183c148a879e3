"""Seeded synthetic inputs for the paged-decode workloads.

Workload i draws from ``numpy.random.default_rng`` streams spawned from
``SeedSequence(1000 + i)``: one child stream each for context lengths, block
tables, pool values, queries and the new tokens' keys and values.  bf16
values are float32 draws from N(0, 1) rounded to bfloat16 with
round-to-nearest-even and kept as raw uint16 bit patterns, so that every
consumer sees exactly the same bits; fp16 values are the same draws converted
to numpy float16 (also round-to-nearest-even).

Pool layout (page 3, mini-infer, "Python Implementation: Physical Block
Pool"): ``[num_blocks, 2 (K/V), layers, kv_heads, block_size, head_dim]``.
Only the attended layer is filled with draws, for every block (used or not);
all other layers stay zero, as the pool there is zero-initialised.

Block tables are ``int32 [S, max_blocks_per_seq]`` with ``-1`` in unused
entries.  For workloads 0, 2, 3 and 4 each sequence takes the next
``ceil(T_b / block_size)`` ids from one random permutation of the pool.
Workload 1 takes its ids from a LIFO free list after a seeded random
allocate/free churn (the free list of the same page's ``BlockPool``), so its
tables are fragmented the way a long-running server's would be.
"""

from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

CONFIG_NAMES = {
    0: "tiny_fp32_mha",
    1: "churned_pool_bf16_gqa7",
    2: "llama8b_decode_bf16",
    3: "long_context_bf16",
    4: "high_concurrency_bf16",
    5: "llama8b_decode_f32",
    6: "llama8b_decode_f16",
    7: "gemma_like_d256_bf16",
    8: "mqa32_decode_bf16",
    9: "mqa32_high_concurrency_bf16",
}

# Sequences' context lengths count the token appended in this step: the new
# token is written at position T_b - 1 and decode then attends over T_b tokens.
_SPECS = {
    0: dict(dtype="f32", S=4, Hq=4, Hkv=4, D=64, BS=16, L=1, layer=0,
            lens=("uniform", 1, 100), NB=64, tables="perm"),
    1: dict(dtype="bf16", S=32, Hq=14, Hkv=2, D=64, BS=16, L=24, layer=11,
            lens=("uniform", 1, 2048), NB=4096, tables="churn"),
    2: dict(dtype="bf16", S=64, Hq=32, Hkv=8, D=128, BS=16, L=1, layer=0,
            lens=("lognormal", 2048.0, 0.5, 128, 8192), NB="1.1x", tables="perm"),
    3: dict(dtype="bf16", S=8, Hq=32, Hkv=8, D=128, BS=32, L=1, layer=0,
            lens=("uniform", 32768, 131072), NB="1.1x", tables="perm"),
    4: dict(dtype="bf16", S=256, Hq=64, Hkv=8, D=128, BS=16, L=1, layer=0,
            lens=("bimodal", 0.7, (16, 512), (4096, 16384)), NB="1.1x", tables="perm"),
    # the Llama-8B-shaped layer of workload 2 with an fp32 cache
    5: dict(dtype="f32", S=64, Hq=32, Hkv=8, D=128, BS=16, L=1, layer=0,
            lens=("lognormal", 2048.0, 0.5, 128, 8192), NB="1.1x", tables="perm"),
    # ... and with an fp16 cache
    6: dict(dtype="f16", S=64, Hq=32, Hkv=8, D=128, BS=16, L=1, layer=0,
            lens=("lognormal", 2048.0, 0.5, 128, 8192), NB="1.1x", tables="perm"),
    # other head shapes on the same length mixes: head_dim 256 with 16 query /
    # 8 KV heads (a Gemma-2-9B-shaped layer), and one KV head shared by 32
    # query heads (multi-query attention) on workload 2's and 4's lengths
    7: dict(dtype="bf16", S=64, Hq=16, Hkv=8, D=256, BS=16, L=1, layer=0,
            lens=("lognormal", 2048.0, 0.5, 128, 8192), NB="1.1x", tables="perm"),
    8: dict(dtype="bf16", S=64, Hq=32, Hkv=1, D=128, BS=16, L=1, layer=0,
            lens=("lognormal", 2048.0, 0.5, 128, 8192), NB="1.1x", tables="perm"),
    9: dict(dtype="bf16", S=256, Hq=32, Hkv=1, D=128, BS=16, L=1, layer=0,
            lens=("bimodal", 0.7, (16, 512), (4096, 16384)), NB="1.1x", tables="perm"),
}

_CHURN_STEPS = 20000
_CHURN_P_ALLOC = 0.55
_POOL_CHUNK_BLOCKS = 256


def config_spec(i: int) -> dict:
    return dict(_SPECS[i])


def bf16_round_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even.

    Inputs are finite draws; NaN/Inf handling is not needed here.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


@dataclass
class Workload:
    """One seeded batch.  Array dtypes: float32 values for ``f32`` workloads,
    uint16 bfloat16 bit patterns for ``bf16`` workloads."""

    index: int
    name: str
    dtype: str
    S: int
    Hq: int
    Hkv: int
    D: int
    BS: int
    L: int
    layer: int
    NB: int
    MB: int
    scale: float
    context_lens: np.ndarray   # int32 [S], includes the appended token
    block_tables: np.ndarray   # int32 [S, MB], -1 where unused
    q: np.ndarray              # [S, Hq, D]
    k_new: np.ndarray          # [S, Hkv, D]
    v_new: np.ndarray          # [S, Hkv, D]
    pool: np.ndarray | None    # [NB, 2, L, Hkv, BS, D] (None if not generated)
    meta: dict = field(default_factory=dict)

    @property
    def positions(self) -> np.ndarray:
        """Token index the new K/V is written to, per sequence."""
        return (self.context_lens - 1).astype(np.int32)

    @property
    def max_len(self) -> int:
        return int(self.context_lens.max()) if self.S else 0

    @property
    def np_dtype(self):
        return {"f32": np.float32, "f16": np.float16}.get(self.dtype, np.uint16)

    def kv_bytes(self) -> int:
        e = 4 if self.dtype == "f32" else 2
        return int(2 * int(self.context_lens.astype(np.int64).sum()) * self.Hkv * self.D * e)


def _draw_lens(rng: np.random.Generator, spec, S: int) -> np.ndarray:
    kind = spec[0]
    if kind == "uniform":
        lo, hi = spec[1], spec[2]
        t = rng.integers(lo, hi + 1, size=S)
    elif kind == "lognormal":
        median, sigma, lo, hi = spec[1:]
        t = np.rint(np.exp(rng.normal(math.log(median), sigma, size=S)))
        t = np.clip(t, lo, hi)
    elif kind == "bimodal":
        frac, (alo, ahi), (blo, bhi) = spec[1], spec[2], spec[3]
        pick_short = rng.random(S) < frac
        short = rng.integers(alo, ahi + 1, size=S)
        long_ = rng.integers(blo, bhi + 1, size=S)
        t = np.where(pick_short, short, long_)
    else:
        raise ValueError(kind)
    return t.astype(np.int32)


def _max_len_of(spec) -> int:
    kind = spec[0]
    if kind == "uniform":
        return spec[2]
    if kind == "lognormal":
        return spec[4]
    if kind == "bimodal":
        return spec[3][1]
    raise ValueError(kind)


def _blocks_needed(lens: np.ndarray, bs: int) -> np.ndarray:
    return (lens.astype(np.int64) + bs - 1) // bs


def _tables_from_perm(rng, lens, bs, nb, mb) -> np.ndarray:
    need = _blocks_needed(lens, bs)
    perm = rng.permutation(nb).astype(np.int32)
    tables = np.full((len(lens), mb), -1, dtype=np.int32)
    off = 0
    for b, n in enumerate(need):
        tables[b, :n] = perm[off:off + n]
        off += n
    assert off <= nb
    return tables


def _tables_after_churn(rng, lens, bs, nb, mb) -> np.ndarray:
    """Fragment a LIFO free list with random allocate/free traffic, then hand
    out the real tables round-robin, one block per sequence per turn."""
    free = list(range(nb))
    held: list[int] = []
    for _ in range(_CHURN_STEPS):
        if free and (not held or rng.random() < _CHURN_P_ALLOC):
            held.append(free.pop())
        elif held:
            i = int(rng.integers(len(held)))
            held[i], held[-1] = held[-1], held[i]
            free.append(held.pop())
    for i in rng.permutation(len(held)):
        free.append(held[int(i)])
    need = _blocks_needed(lens, bs)
    tables = np.full((len(lens), mb), -1, dtype=np.int32)
    have = np.zeros(len(lens), dtype=np.int64)
    while (have < need).any():
        for b in range(len(lens)):
            if have[b] < need[b]:
                tables[b, have[b]] = free.pop()
                have[b] += 1
    return tables


def _normal_values(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    """float32 draws; bf16 as RNE-rounded bit patterns; fp16 as numpy float16
    (numpy's float32 -> float16 conversion rounds to nearest even)."""
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if dtype == "f32":
        return x
    if dtype == "f16":
        return x.astype(np.float16)
    return bf16_round_bits(x)


def storage_dtype(dtype: str):
    """numpy array type of a pool dtype's raw storage."""
    return {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}[dtype]


def _fill_pool(seed_seq: np.random.SeedSequence, nb, L, layer, hkv, bs, d, dtype,
               threads: int | None) -> np.ndarray:
    npdt = storage_dtype(dtype)
    pool = np.zeros((nb, 2, L, hkv, bs, d), dtype=npdt)
    nchunks = (nb + _POOL_CHUNK_BLOCKS - 1) // _POOL_CHUNK_BLOCKS
    children = seed_seq.spawn(max(nchunks, 1))

    def work(c):
        lo = c * _POOL_CHUNK_BLOCKS
        hi = min(nb, lo + _POOL_CHUNK_BLOCKS)
        rng = np.random.default_rng(children[c])
        pool[lo:hi, :, layer] = _normal_values(rng, (hi - lo, 2, hkv, bs, d), dtype)

    nthreads = threads or min(16, os.cpu_count() or 1)
    if nchunks <= 1 or nthreads <= 1:
        for c in range(nchunks):
            work(c)
    else:
        with ThreadPoolExecutor(nthreads) as ex:
            list(ex.map(work, range(nchunks)))
    return pool


def make_workload(index: int, *, with_pool: bool = True, seed_offset: int = 0,
                  keep_lens: bool = False, threads: int | None = None, **overrides) -> Workload:
    """Build workload ``index`` (0..9).

    ``overrides`` replaces spec entries (e.g. ``S=8`` for a reduced batch of
    the same shape family); ``seed_offset`` selects an independent replica
    (used to rotate inputs so that timed runs do not hit in cache).  With
    ``keep_lens`` the replica keeps replica 0's context lengths (so the same
    bytes are moved) and redraws only tables, pool values, q and new rows.
    """
    spec = config_spec(index)
    spec.update(overrides)
    ss = np.random.SeedSequence(1000 + index + 7919 * seed_offset)
    s_lens, s_tab, s_pool, s_q, s_k, s_v = ss.spawn(6)
    if keep_lens:
        s_lens = np.random.SeedSequence(1000 + index).spawn(6)[0]
    S, Hq, Hkv, D, BS = spec["S"], spec["Hq"], spec["Hkv"], spec["D"], spec["BS"]
    L, layer, dtype = spec["L"], spec["layer"], spec["dtype"]

    lens = spec.get("context_lens")
    if lens is None:
        lens = _draw_lens(np.random.default_rng(s_lens), spec["lens"], S)
    lens = np.asarray(lens, dtype=np.int32)
    mb = spec.get("MB") or max(1, -(-_max_len_of(spec["lens"]) // BS))
    total_blocks = int(_blocks_needed(lens, BS).sum())
    nb = spec["NB"]
    if nb == "1.1x":
        nb = max(1, math.ceil(1.1 * total_blocks))
    if total_blocks > nb:
        raise ValueError(f"pool of {nb} blocks cannot hold {total_blocks}")

    rng_t = np.random.default_rng(s_tab)
    if spec["tables"] == "perm":
        tables = _tables_from_perm(rng_t, lens, BS, nb, mb)
    elif spec["tables"] == "churn":
        tables = _tables_after_churn(rng_t, lens, BS, nb, mb)
    else:
        raise ValueError(spec["tables"])

    q = _normal_values(np.random.default_rng(s_q), (S, Hq, D), dtype)
    k_new = _normal_values(np.random.default_rng(s_k), (S, Hkv, D), dtype)
    v_new = _normal_values(np.random.default_rng(s_v), (S, Hkv, D), dtype)
    pool = _fill_pool(s_pool, nb, L, layer, Hkv, BS, D, dtype, threads) if with_pool else None

    return Workload(
        index=index, name=CONFIG_NAMES.get(index, f"workload{index}"), dtype=dtype,
        S=S, Hq=Hq, Hkv=Hkv, D=D, BS=BS, L=L, layer=layer, NB=nb, MB=mb,
        scale=float(1.0 / math.sqrt(D)), context_lens=lens, block_tables=tables,
        q=q, k_new=k_new, v_new=v_new, pool=pool,
        meta=dict(spec=spec, total_blocks=total_blocks, seed=1000 + index,
                  seed_offset=seed_offset),
    )


@dataclass
class AppendBatch:
    """Inputs of the two multi-row appends (all layers of one token; several
    tokens of one layer), with a pool whose background is random bits so
    that any stray or missing write changes bytes a test compares."""

    dtype: str
    S: int
    Hkv: int
    D: int
    BS: int
    L: int
    layer: int
    NB: int
    MB: int
    pool: np.ndarray             # [NB, 2, L, Hkv, BS, D]
    block_tables: np.ndarray     # int32 [S, MB], -1 where unused
    start_positions: np.ndarray  # int32 [S], first new position (negative = skip)
    token_offsets: np.ndarray    # int32 [S + 1], rows of sequence b: [off[b], off[b+1])
    k_rows: np.ndarray           # [N, Hkv, D] new rows, N = token_offsets[-1]
    v_rows: np.ndarray
    k_layers: np.ndarray         # [S, L, Hkv, D] one token for every layer
    v_layers: np.ndarray

    @property
    def total_rows(self) -> int:
        return int(self.token_offsets[-1])


def make_append_batch(seed: int, *, dtype: str, Hkv: int, D: int, BS: int, L: int, layer: int,
                      starts, counts, spare_blocks: int = 3) -> AppendBatch:
    """Sequence b gets counts[b] new tokens from position starts[b] on (the
    layered rows are for position starts[b] alone).  Its table holds
    ceil((starts[b] + max(counts[b], 1)) / BS) blocks drawn from one random
    permutation of the pool; a negative start gets one block and is skipped
    by the appends."""
    starts = np.asarray(starts, dtype=np.int32)
    counts = np.asarray(counts, dtype=np.int64)
    S = len(starts)
    ends = np.where(starts >= 0, starts.astype(np.int64) + np.maximum(counts, 1), 1)
    need = (ends + BS - 1) // BS
    mb = max(1, int(need.max()) if S else 1)
    nb = int(need.sum()) + spare_blocks
    ss = np.random.SeedSequence(seed)
    s_tab, s_pool, s_rows, s_layers = ss.spawn(4)
    perm = np.random.default_rng(s_tab).permutation(nb).astype(np.int32)
    tables = np.full((S, mb), -1, dtype=np.int32)
    off = 0
    for b in range(S):
        n = int(need[b])
        tables[b, :n] = perm[off:off + n]
        off += n
    npdt = storage_dtype(dtype)
    shape = (nb, 2, L, Hkv, BS, D)
    nbytes = int(np.prod(shape)) * np.dtype(npdt).itemsize
    pool = np.frombuffer(np.random.default_rng(s_pool).bytes(nbytes), dtype=npdt)
    pool = pool.reshape(shape).copy()
    offsets = np.zeros(S + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    n_rows = int(offsets[-1])
    rng_r = np.random.default_rng(s_rows)
    k_rows = _normal_values(rng_r, (n_rows, Hkv, D), dtype)
    v_rows = _normal_values(rng_r, (n_rows, Hkv, D), dtype)
    rng_l = np.random.default_rng(s_layers)
    k_layers = _normal_values(rng_l, (S, L, Hkv, D), dtype)
    v_layers = _normal_values(rng_l, (S, L, Hkv, D), dtype)
    return AppendBatch(dtype=dtype, S=S, Hkv=Hkv, D=D, BS=BS, L=L, layer=layer, NB=nb, MB=mb,
                       pool=pool, block_tables=tables, start_positions=starts,
                       token_offsets=offsets, k_rows=k_rows, v_rows=v_rows,
                       k_layers=k_layers, v_layers=v_layers)
