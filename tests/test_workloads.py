"""The seeded generators: deterministic, well-formed, and shaped like the
decode workloads (pool geometry, length mix, fragmented tables)."""

import math

import numpy as np
import pytest

from workloads import bf16_round_bits, make_workload


@pytest.mark.parametrize("i", range(10))
def test_metadata_well_formed(i):
    w = make_workload(i, with_pool=False)
    assert w.block_tables.shape == (w.S, w.MB)
    assert w.context_lens.min() >= 1
    assert w.context_lens.max() <= w.MB * w.BS
    used = []
    for b in range(w.S):
        n = math.ceil(int(w.context_lens[b]) / w.BS)
        row = w.block_tables[b]
        assert (row[:n] >= 0).all() and (row[:n] < w.NB).all()
        assert (row[n:] == -1).all()
        used.extend(row[:n].tolist())
    assert len(used) == len(set(used)), "two sequences share a physical block"
    assert w.Hq % w.Hkv == 0
    assert w.q.shape == (w.S, w.Hq, w.D)


def test_deterministic():
    a = make_workload(1)
    b = make_workload(1)
    assert a.pool.tobytes() == b.pool.tobytes()
    assert a.block_tables.tobytes() == b.block_tables.tobytes()
    assert a.q.tobytes() == b.q.tobytes()
    c = make_workload(1, seed_offset=1, with_pool=False)
    assert c.q.tobytes() != a.q.tobytes()


def test_thread_count_does_not_change_values():
    a = make_workload(0, threads=1)
    b = make_workload(0, threads=8)
    assert a.pool.tobytes() == b.pool.tobytes()


def test_shapes_of_named_workloads():
    w1 = make_workload(1, with_pool=False)
    assert (w1.NB, w1.L, w1.Hkv, w1.BS, w1.D, w1.Hq, w1.S, w1.layer) == (4096, 24, 2, 16, 64, 14, 32, 11)
    w2 = make_workload(2, with_pool=False)
    assert (w2.Hq, w2.Hkv, w2.D, w2.BS, w2.S) == (32, 8, 128, 16, 64)
    assert w2.context_lens.min() >= 128 and w2.context_lens.max() <= 8192
    assert w2.NB == math.ceil(1.1 * w2.meta["total_blocks"])
    w3 = make_workload(3, with_pool=False)
    assert w3.BS == 32 and w3.context_lens.min() >= 32768 and w3.context_lens.max() <= 131072
    w4 = make_workload(4, with_pool=False)
    short = (w4.context_lens <= 512).mean()
    assert 0.55 < short < 0.85


def test_churned_tables_are_fragmented():
    w = make_workload(1, with_pool=False)
    row = w.block_tables[0][: math.ceil(int(w.context_lens[0]) / 16)]
    steps = np.diff(row.astype(np.int64))
    assert (steps != -1).mean() > 0.5, "tables look like a fresh LIFO run"


def test_bf16_rounding_is_rne():
    x = np.array([1.0, 1.00390625, 1.01171875, -2.5, 3.140625], np.float32)
    # 1 + 2^-8 is a tie between 1.0 and 1 + 2^-7: even mantissa wins (1.0).
    # 1 + 3*2^-8 is a tie between 1+2^-7 and 1+2^-6: even wins (1+2^-6).
    assert bf16_round_bits(x).tolist() == [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x4049]


def test_append_batch_well_formed():
    from workloads import make_append_batch
    starts = [0, 5, -1, 16, 0]
    counts = [33, 4, 3, 0, 1]
    a = make_append_batch(5, dtype="bf16", Hkv=2, D=64, BS=16, L=3, layer=1,
                          starts=starts, counts=counts)
    b = make_append_batch(5, dtype="bf16", Hkv=2, D=64, BS=16, L=3, layer=1,
                          starts=starts, counts=counts)
    assert a.pool.tobytes() == b.pool.tobytes() and a.k_rows.tobytes() == b.k_rows.tobytes()
    assert a.token_offsets.tolist() == [0, 33, 37, 40, 40, 41]
    assert a.k_rows.shape == (41, 2, 64) and a.k_layers.shape == (5, 3, 2, 64)
    used = a.block_tables[a.block_tables >= 0]
    assert len(used) == len(set(used.tolist())) and used.max() < a.NB
    for s, n, row in zip(starts, counts, a.block_tables):
        if s >= 0:   # every position the appends write has a block
            assert (row[:math.ceil((s + max(n, 1)) / 16)] >= 0).all()
