"""Pins for the CPU oracle: each check ties an oracle function to something
other than itself (the pages' worked examples, a library routine, brute
force, closed forms, exact invariants).  ``test_mutants_are_caught`` plants
plausible mistakes in the oracle (on the CPU) and confirms that some pin
fails for every one of them.
"""

from __future__ import annotations

import math
from unittest import mock

import numpy as np
import pytest
import torch

import oracle
import oracle.paged as P
from workloads import bf16_round_bits, make_workload

from conftest import read_golden

# ----------------------------------------------------------------------------
# helpers written for the tests (independent of the oracle's code)
# ----------------------------------------------------------------------------


def _bf16_to_f64_via_torch(bits: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(bits.astype(np.uint16).view(np.int16)).view(torch.bfloat16)
    return t.to(torch.float64).numpy()


def _scatter_contiguous(pool, layer, table_row, K, V, bs):
    """Place a contiguous sequence into its blocks, one block-sized slice at
    a time (block j of the table holds tokens j*bs .. j*bs+bs-1)."""
    T = K.shape[0]
    for j in range(math.ceil(T / bs)):
        n = min(bs, T - j * bs)
        pool[table_row[j], 0, layer, :, :n, :] = np.swapaxes(K[j * bs:j * bs + n], 0, 1)
        pool[table_row[j], 1, layer, :, :n, :] = np.swapaxes(V[j * bs:j * bs + n], 0, 1)


def _random_paged_case(rng, *, S, Hq, Hkv, D, BS, L, layer, max_T, dtype, poison=True):
    """Contiguous per-sequence K/V (the ground truth), scattered into a pool
    through random distinct block ids; unused storage poisoned with NaN."""
    lens = rng.integers(0, max_T + 1, size=S).astype(np.int32)
    lens[0] = max_T
    need = [math.ceil(int(t) / BS) for t in lens]
    MB = max(1, max(need))
    NB = sum(need) + 5
    ids = rng.permutation(NB).astype(np.int32)
    tables = np.full((S, MB), -1, np.int32)
    off = 0
    for b in range(S):
        tables[b, :need[b]] = ids[off:off + need[b]]
        off += need[b]
    if dtype == "f32":
        store = np.float32
        nan = np.float32(np.nan)
        draw = lambda shape: rng.standard_normal(shape).astype(np.float32)  # noqa: E731
    elif dtype == "f16":
        store = np.float16
        nan = np.float16(np.nan)
        draw = lambda shape: rng.standard_normal(shape).astype(np.float16)  # noqa: E731
    else:
        store = np.uint16
        nan = np.uint16(0x7FC0)
        draw = lambda shape: bf16_round_bits(rng.standard_normal(shape).astype(np.float32))  # noqa: E731
    pool = np.full((NB, 2, L, Hkv, BS, D), nan if poison else 0, dtype=store)
    Ks, Vs = [], []
    for b in range(S):
        K = draw((int(lens[b]), Hkv, D))
        V = draw((int(lens[b]), Hkv, D))
        _scatter_contiguous(pool, layer, tables[b], K, V, BS)
        Ks.append(K)
        Vs.append(V)
    if poison:
        tables = tables.copy()
        for b in range(S):
            tables[b, need[b]:] = 2**31 - 1   # garbage padding, never read
    q = draw((S, Hq, D))
    return dict(pool=pool, tables=tables, lens=lens, q=q, Ks=Ks, Vs=Vs, MB=MB, NB=NB)


def _to_f64(x, dtype):
    if dtype == "f16":   # through torch's half type, not numpy's
        return torch.from_numpy(np.ascontiguousarray(x)).to(torch.float64).numpy()
    return x.astype(np.float64) if dtype == "f32" else _bf16_to_f64_via_torch(x)


def _half_value_from_bits(u: int) -> float:
    """IEEE 754 binary16 from its definition: sign, 5-bit exponent with bias
    15, 10-bit fraction; exponent 0 is subnormal (no implicit 1)."""
    sign = -1.0 if u >> 15 else 1.0
    e = (u >> 10) & 0x1F
    f = u & 0x3FF
    if e == 0:
        return sign * f * 2.0 ** -24
    return sign * (1024 + f) * 2.0 ** (e - 25)


def _sdpa_reference(q, K, V, scale):
    """torch's scaled_dot_product_attention in float64, KV heads repeated to
    the query head count in contiguous groups."""
    Hq, D = q.shape
    T, Hkv, _ = K.shape
    if T == 0:
        return np.zeros((Hq, D))
    G = Hq // Hkv
    qt = torch.from_numpy(q).reshape(1, Hq, 1, D)
    kt = torch.from_numpy(np.ascontiguousarray(np.swapaxes(K, 0, 1))).repeat_interleave(G, dim=0)[None]
    vt = torch.from_numpy(np.ascontiguousarray(np.swapaxes(V, 0, 1))).repeat_interleave(G, dim=0)[None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)
    return o.reshape(Hq, D).numpy()


# ----------------------------------------------------------------------------
# pin checks (plain functions so the mutation test can rerun them)
# ----------------------------------------------------------------------------


def check_resolve_page_examples():
    tables = {"A": np.array([14, 89, 3], np.int32), "B": np.array([4, 1, 7], np.int32)}
    for name, t, expected in read_golden("resolve_page_examples.txt"):
        slots = oracle.resolve_slots(tables[name][None], np.array([41], np.int32), 16, 48)
        assert slots[0, int(t)] == int(expected), (name, t, slots[0, int(t)], expected)


def check_gather_coordinate_pool():
    shape = (8, 2, 2, 2, 4, 2)
    pool = np.arange(np.prod(shape), dtype=np.float32).reshape(shape)
    table = np.array([[4, 1, 7]], np.int32)
    k, v, mask = oracle.paged_kv_gather(pool, 1, table, np.array([10], np.int32), 12)
    for kv, t, g, d, expected in read_golden("gather_coordinate_pool.txt"):
        src = k if kv == "0" else v
        assert src[0, int(t), int(g), int(d)] == float(expected), (kv, t, g, d)
    assert mask[0].tolist() == [1] * 10 + [0, 0]
    assert not k[0, 10:].any() and not v[0, 10:].any()


def check_contiguous_equivalence(dtype):
    rng = np.random.default_rng(11)
    c = _random_paged_case(rng, S=5, Hq=6, Hkv=2, D=8, BS=4, L=3, layer=2, max_T=23, dtype=dtype)
    for b in range(5):
        K, V = oracle.gather_sequence(c["pool"], 2, c["tables"][b], int(c["lens"][b]))
        assert K.tobytes() == c["Ks"][b].tobytes()
        assert V.tobytes() == c["Vs"][b].tobytes()
    k, v, mask = oracle.paged_kv_gather(c["pool"], 2, c["tables"], c["lens"], int(c["lens"].max()))
    for b in range(5):
        T = int(c["lens"][b])
        assert k[b, :T].tobytes() == c["Ks"][b].tobytes()
        assert v[b, :T].tobytes() == c["Vs"][b].tobytes()
        assert mask[b].sum() == T


def check_attention_vs_sdpa(dtype):
    rng = np.random.default_rng(12)
    c = _random_paged_case(rng, S=6, Hq=8, Hkv=2, D=16, BS=4, L=2, layer=1, max_T=37, dtype=dtype)
    scale = 0.3
    out = oracle.paged_attention_decode(c["pool"], dtype, 1, c["tables"], c["lens"], c["q"], scale)
    s64 = float(np.float32(scale))
    for b in range(6):
        ref = _sdpa_reference(_to_f64(c["q"][b], dtype), _to_f64(c["Ks"][b], dtype),
                              _to_f64(c["Vs"][b], dtype), s64)
        np.testing.assert_allclose(out[b], ref, rtol=1e-12, atol=1e-12)


def check_bruteforce_tiny():
    """Per-element Python loops with math.exp on small integer inputs."""
    rng = np.random.default_rng(13)
    for D in (1, 2):
        for BS in (1, 2, 4):
            for T in range(0, 6):
                Hq, Hkv = 4, 2
                K = rng.integers(-3, 4, size=(T, Hkv, D)).astype(np.float32)
                V = rng.integers(-3, 4, size=(T, Hkv, D)).astype(np.float32)
                q = rng.integers(-2, 3, size=(1, Hq, D)).astype(np.float32)
                nblk = math.ceil(T / BS)
                NB = nblk + 3
                table = np.full((1, max(nblk, 1)), -1, np.int32)
                table[0, :nblk] = rng.permutation(NB)[:nblk]
                pool = np.full((NB, 2, 1, Hkv, BS, D), np.nan, np.float32)
                _scatter_contiguous(pool, 0, table[0], K, V, BS)
                got = oracle.paged_attention_decode(pool, "f32", 0, table, np.array([T], np.int32), q, 0.5)
                for h in range(Hq):
                    g = h // (Hq // Hkv)
                    for d in range(D):
                        if T == 0:
                            want = 0.0
                        else:
                            s = [0.5 * sum(float(q[0, h, i]) * float(K[t, g, i]) for i in range(D)) for t in range(T)]
                            m = max(s)
                            w = [math.exp(x - m) for x in s]
                            want = sum(w[t] * float(V[t, g, d]) for t in range(T)) / sum(w)
                        assert abs(got[0, h, d] - want) <= 1e-12 * max(1.0, abs(want)), (D, BS, T, h, d)


def check_closed_forms():
    rng = np.random.default_rng(14)
    Hq, Hkv, D = 4, 4, 5
    q = rng.standard_normal((Hq, D))
    # T = 1: the only weight is 1, so the output is that token's V row.
    K = rng.standard_normal((1, Hkv, D))
    V = rng.standard_normal((1, Hkv, D))
    np.testing.assert_array_equal(oracle.attend(q, K, V, 0.7), V[0])
    # scale = 0: uniform weights, the output is the mean of the V rows.
    K = rng.standard_normal((7, Hkv, D))
    V = rng.standard_normal((7, Hkv, D))
    np.testing.assert_allclose(oracle.attend(q, K, V, 0.0), V.mean(axis=0), rtol=0, atol=1e-14)
    # T = 2: V0 + sigmoid(s1 - s0) * (V1 - V0).
    K = rng.standard_normal((2, Hkv, D))
    V = rng.standard_normal((2, Hkv, D))
    sc = 0.37
    got = oracle.attend(q, K, V, sc)
    for h in range(Hq):
        s0 = sc * float(q[h] @ K[0, h])
        s1 = sc * float(q[h] @ K[1, h])
        sig = 1.0 / (1.0 + math.exp(-(s1 - s0)))
        np.testing.assert_allclose(got[h], V[0, h] + sig * (V[1, h] - V[0, h]), rtol=0, atol=1e-14)


def check_invariants():
    rng = np.random.default_rng(15)
    Hq, Hkv, D, T = 6, 3, 8, 29
    q = rng.standard_normal((Hq, D))
    K = rng.standard_normal((T, Hkv, D))
    V = rng.standard_normal((T, Hkv, D))
    out = oracle.attend(q, K, V, 0.4)
    # convex combination of the V rows of the head's KV group
    for h in range(Hq):
        g = h // (Hq // Hkv)
        assert np.all(out[h] <= V[:, g].max(axis=0) + 1e-12)
        assert np.all(out[h] >= V[:, g].min(axis=0) - 1e-12)
    # adding one vector to every K row shifts all scores of a head equally
    u = rng.standard_normal((Hkv, D))
    np.testing.assert_allclose(oracle.attend(q, K + u, V, 0.4), out, rtol=0, atol=1e-12)
    # adding one vector to every V row adds it to the output
    c = rng.standard_normal((Hkv, D))
    shifted = oracle.attend(q, K, V + c, 0.4)
    for h in range(Hq):
        np.testing.assert_allclose(shifted[h], out[h] + c[h // (Hq // Hkv)], rtol=0, atol=1e-12)


def check_block_permutation_invariance():
    """Relabelling physical blocks (and the tables with them) changes
    nothing, bit for bit."""
    w = make_workload(0)
    rng = np.random.default_rng(16)
    perm = rng.permutation(w.NB)
    pool2 = np.empty_like(w.pool)
    pool2[perm] = w.pool
    tables2 = np.where(w.block_tables >= 0, perm[np.maximum(w.block_tables, 0)], -1).astype(np.int32)
    a = oracle.paged_attention_decode(w.pool, w.dtype, w.layer, w.block_tables, w.context_lens, w.q, w.scale)
    b = oracle.paged_attention_decode(pool2, w.dtype, w.layer, tables2, w.context_lens, w.q, w.scale)
    assert a.tobytes() == b.tobytes()
    ga = oracle.paged_kv_gather(w.pool, w.layer, w.block_tables, w.context_lens, w.max_len)
    gb = oracle.paged_kv_gather(pool2, w.layer, tables2, w.context_lens, w.max_len)
    for x, y in zip(ga, gb):
        assert x.tobytes() == y.tobytes()


def check_append_fixture():
    pool = np.zeros((8, 2, 2, 2, 4, 2), np.float32)
    table = np.array([[4, 1, 7]], np.int32)
    k_new = np.array([[[1, 2], [3, 4]]], np.float32)
    v_new = np.array([[[5, 6], [7, 8]]], np.float32)
    out = oracle.kv_append(pool, 0, table, np.array([6], np.int32), k_new, v_new)
    flat = out.reshape(-1)
    expected = {int(i): float(v) for i, v in read_golden("append_example.txt")}
    nz = {int(i): float(flat[i]) for i in np.flatnonzero(flat)}
    assert nz == expected, (nz, expected)
    assert not pool.any()   # not in place by default


def check_append_layers_fixture():
    pool = np.zeros((8, 2, 2, 2, 4, 2), np.float32)
    table = np.array([[4, 1, 7]], np.int32)
    k_new = np.array([[[[1, 2], [3, 4]], [[9, 10], [11, 12]]]], np.float32)
    v_new = np.array([[[[5, 6], [7, 8]], [[13, 14], [15, 16]]]], np.float32)
    out = oracle.kv_append_layers(pool, table, np.array([6], np.int32), k_new, v_new)
    flat = out.reshape(-1)
    expected = {int(i): float(v) for i, v in read_golden("append_layers_example.txt")}
    nz = {int(i): float(flat[i]) for i in np.flatnonzero(flat)}
    assert nz == expected, (nz, expected)
    assert not pool.any()


def check_append_tokens_fixture():
    pool = np.zeros((8, 2, 1, 1, 2, 1), np.float32)
    tables = np.array([[3, 5], [6, 2]], np.int32)
    k_new = np.array([1, 2, 3, 4, 5], np.float32).reshape(5, 1, 1)
    v_new = k_new + 10
    out = oracle.kv_append_tokens(pool, 0, tables, np.array([1, 0], np.int32),
                                  np.array([0, 3, 5], np.int32), k_new, v_new)
    flat = out.reshape(-1)
    expected = {int(i): float(v) for i, v in read_golden("append_tokens_example.txt")}
    nz = {int(i): float(flat[i]) for i in np.flatnonzero(flat)}
    assert nz == expected, (nz, expected)
    assert not pool.any()


def check_multi_appends_equal_single_appends():
    """The all-layer append equals one kv_append per layer, and the prompt
    append equals one kv_append per token offset."""
    rng = np.random.default_rng(23)
    NB, L, H, BS, D, S = 24, 3, 2, 4, 3, 3
    pool = rng.standard_normal((NB, 2, L, H, BS, D)).astype(np.float32)
    tables = rng.permutation(NB)[:S * 6].reshape(S, 6).astype(np.int32)
    pos = np.array([5, -1, 17], np.int32)
    k_l = rng.standard_normal((S, L, H, D)).astype(np.float32)
    v_l = rng.standard_normal((S, L, H, D)).astype(np.float32)
    ref = pool.copy()
    for layer in range(L):
        ref = oracle.kv_append(ref, layer, tables, pos, k_l[:, layer], v_l[:, layer])
    assert oracle.kv_append_layers(pool, tables, pos, k_l, v_l).tobytes() == ref.tobytes()
    starts = np.array([0, 7, -2], np.int32)
    counts = np.array([9, 4, 3], np.int32)
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    k_t = rng.standard_normal((int(offs[-1]), H, D)).astype(np.float32)
    v_t = rng.standard_normal((int(offs[-1]), H, D)).astype(np.float32)
    ref = pool.copy()
    for i in range(int(counts.max())):
        p_i = np.where((starts >= 0) & (i < counts), starts + i, -1).astype(np.int32)
        rows = np.minimum(offs[:-1] + i, offs[-1] - 1)
        ref = oracle.kv_append(ref, 2, tables, p_i, k_t[rows], v_t[rows])
    got = oracle.kv_append_tokens(pool, 2, tables, starts, offs, k_t, v_t)
    assert got.tobytes() == ref.tobytes()


def check_append_then_gather():
    rng = np.random.default_rng(17)
    c = _random_paged_case(rng, S=4, Hq=2, Hkv=2, D=4, BS=4, L=2, layer=1, max_T=13,
                           dtype="bf16", poison=False)
    lens = np.maximum(c["lens"], 1)
    pos = (lens - 1).astype(np.int32)
    # make sure every tail block exists in the table
    tables = c["tables"].copy()
    k_new = bf16_round_bits(rng.standard_normal((4, 2, 4)).astype(np.float32))
    v_new = bf16_round_bits(rng.standard_normal((4, 2, 4)).astype(np.float32))
    for b in range(4):
        if c["lens"][b] == 0:
            tables[b, 0] = c["NB"] - 1 - b
    out = oracle.kv_append(c["pool"], 1, tables, pos, k_new, v_new)
    k, v, _ = oracle.paged_kv_gather(out, 1, tables, lens, int(lens.max()))
    for b in range(4):
        assert k[b, pos[b]].tobytes() == k_new[b].tobytes()
        assert v[b, pos[b]].tobytes() == v_new[b].tobytes()
    changed = np.flatnonzero((out != c["pool"]).reshape(-1))
    assert len(changed) <= 4 * 2 * 2 * 4


def check_waste_examples():
    for row in read_golden("waste_examples.txt"):
        kind = row[0]
        if kind == "naive":
            r = oracle.naive_waste_ratio(int(row[1]), int(row[2]))
            assert r == float(row[3]) and f"{100 * r:.1f}%" == "97.9%"
        elif kind == "bound":
            b = oracle.paged_waste_bound(int(row[1]), int(row[2]))
            assert b == float(row[3]) and b < float(row[4])
            assert oracle.paged_waste_ratio(int(row[1]), int(row[2])) <= b
        elif kind == "paged":
            assert oracle.paged_waste_slots(int(row[1]), int(row[2])) == int(row[3]), row
    for bs in (16, 32):
        for n in range(1, 10001):
            w = oracle.paged_waste_slots(n, bs)
            assert 0 <= w <= bs - 1
            assert oracle.paged_waste_ratio(n, bs) <= oracle.paged_waste_bound(n, bs) < bs / n


def check_free_stack():
    st = oracle.FreeBlockStack(5)
    got = [st.allocate() for _ in range(5)]
    assert got == [4, 3, 2, 1, 0]
    with pytest.raises(MemoryError):
        st.allocate()
    st.free(2)
    st.free(0)
    assert st.allocate() == 0 and st.allocate() == 2


def check_block_manager_page_figures():
    """[mini-infer] "The Problem" / "Memory Waste Analysis" with B = 16: a
    42-token request holds 3 blocks (48 slots, 6 wasted); a 400-token one
    holds 25 blocks and wastes nothing; one more token opens block 26 and the
    waste reaches the page's maximum B - 1 = 15."""
    m = oracle.BlockManagerModel(num_blocks=64, block_size=16, max_blocks_per_seq=32)
    m.add_sequence(1)
    m.add_sequence(2)
    assert m.reserve([1, 2], [42, 400]) == [0, 0]
    st = m.stats()
    assert (len(m.tables[1]), len(m.tables[2])) == (3, 25)
    assert (st["blocks_used"], st["tokens"], st["slots"], st["waste_slots"]) == (28, 442, 448, 6)
    assert m.blocks_needed([2], [1]) == 1
    assert m.reserve([2], [1]) == [400]
    assert m.stats()["waste_slots"] == 6 + 15
    assert m.stats()["blocks_free"] == 64 - 29


def check_block_manager_lifo_reuse():
    """The page's stack hands out N-1 first and reuses the last freed block
    first; a finished sequence returns its blocks in logical order (block 0
    first), so its last block is the next handed out.  Hand-derived."""
    m = oracle.BlockManagerModel(num_blocks=8, block_size=16, max_blocks_per_seq=4)
    for s in (1, 2, 3):
        m.add_sequence(s)
    m.reserve([1], [20])                  # 2 blocks: 7, 6
    m.reserve([2], [1])                   # 5
    assert m.tables[1] == [7, 6] and m.tables[2] == [5]
    m.release(1)                          # pushes 7, then 6
    m.reserve([3], [17])                  # pops 6, then 7
    assert m.tables[3] == [6, 7]
    tab, lens = m.block_tables([3, 2])
    assert tab.tolist() == [[6, 7, -1, -1], [5, -1, -1, -1]] and lens.tolist() == [17, 1]
    # one decode token for each: only a sequence whose blocks are all full needs one
    m.add_sequence(4)
    m.reserve([4], [16])                  # 4
    assert m.blocks_needed([2, 3, 4], [1, 1, 1]) == 0 + 0 + 1
    assert m.reserve([2, 3, 4], [1, 1, 1]) == [1, 17, 16]
    assert m.tables[4] == [4, 3]


def check_block_manager_admission():
    """Admission ([kv-cache] section 3.1): a step runs only if the pool holds
    the blocks it needs; otherwise the out-of-blocks error of the page's
    allocator is raised and nothing changes (all or nothing)."""
    m = oracle.BlockManagerModel(num_blocks=4, block_size=4, max_blocks_per_seq=8)
    m.add_sequence(0)
    m.add_sequence(1)
    m.reserve([0], [12])                  # 3 of 4 blocks
    before = (dict(m.lens), {k: list(v) for k, v in m.tables.items()}, len(m.stack))
    assert m.blocks_needed([1, 0], [5, 1]) == 2 + 1
    with pytest.raises(MemoryError):
        m.reserve([1, 0], [5, 1])
    assert (dict(m.lens), {k: list(v) for k, v in m.tables.items()}, len(m.stack)) == before
    with pytest.raises(ValueError):       # wider than a block-table row
        m.reserve([1], [33])
    with pytest.raises(ValueError):       # a sequence twice in one step
        m.reserve([1, 1], [1, 1])
    assert m.reserve([1], [4]) == [0] and len(m.stack) == 0


def check_block_manager_random_invariants():
    """Seeded random traffic: blocks are conserved and never shared, each
    sequence holds exactly the blocks its tokens fill, per-sequence waste
    stays within [0, B - 1] and the total equals the pinned per-sequence
    waste arithmetic."""
    rng = np.random.default_rng(3)
    B, NB = 16, 96
    m = oracle.BlockManagerModel(num_blocks=NB, block_size=B, max_blocks_per_seq=12)
    next_id = 0
    for _ in range(600):
        live = list(m.lens)
        op = rng.random()
        if op < 0.2 or not live:
            m.add_sequence(next_id)
            next_id += 1
        elif op < 0.35:
            m.release(live[int(rng.integers(len(live)))])
        else:
            k = int(rng.integers(1, len(live) + 1))
            seqs = [live[int(i)] for i in rng.permutation(len(live))[:k]]
            counts = [int(rng.integers(0, 20)) if rng.random() < 0.3 else 1 for _ in seqs]
            try:
                m.reserve(seqs, counts)
            except (MemoryError, ValueError):
                pass
        held = [b for t in m.tables.values() for b in t]
        free = [int(x) for x in m.stack._stack[:len(m.stack)]]
        assert len(held) == len(set(held)) and not set(held) & set(free)
        assert sorted(held + free) == list(range(NB))
        for s, t in m.tables.items():
            assert len(t) == math.ceil(m.lens[s] / B)
            assert 0 <= len(t) * B - m.lens[s] <= B - 1
        st = m.stats()
        assert st["waste_slots"] == sum(oracle.paged_waste_slots(n, B) for n in m.lens.values())
        assert st["blocks_free"] + st["blocks_used"] == NB


def check_dense_masked_decode():
    """The gather-then-dense path of [mini-infer] v0.2.0 gives the paged
    decode's result: gathered K/V with the gather's mask through the dense
    decode equal, bit for bit, the paged decode (both take the same rows to
    the same attention); with random non-prefix masks the dense decode
    equals per-element loops over the unmasked rows; and the values of
    masked rows do not matter."""
    rng = np.random.default_rng(21)
    for dtype in ("f32", "bf16", "f16"):
        c = _random_paged_case(rng, S=5, Hq=6, Hkv=2, D=8, BS=4, L=2, layer=1, max_T=19,
                               dtype=dtype)
        max_len = int(c["lens"].max())
        k, v, mask = oracle.paged_kv_gather(c["pool"], 1, c["tables"], c["lens"], max_len)
        dense = oracle.dense_masked_decode(k, v, mask, c["q"], dtype, 0.37)
        paged = oracle.paged_attention_decode(c["pool"], dtype, 1, c["tables"], c["lens"],
                                              c["q"], 0.37)
        assert dense.tobytes() == paged.tobytes()
    S, L, Hq, Hkv, D = 3, 7, 4, 2, 2
    k = rng.integers(-3, 4, size=(S, L, Hkv, D)).astype(np.float32)
    v = rng.integers(-3, 4, size=(S, L, Hkv, D)).astype(np.float32)
    q = rng.integers(-2, 3, size=(S, Hq, D)).astype(np.float32)
    mask = (rng.random((S, L)) < 0.5).astype(np.uint8)
    mask[0] = 0                                   # nothing cached: zero row
    mask[1, 3] = 1
    got = oracle.dense_masked_decode(k, v, mask, q, "f32", 0.5)
    for b in range(S):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            ts = [t for t in range(L) if mask[b, t]]
            if not ts:
                assert not got[b, h].any()
                continue
            sc = [0.5 * sum(float(q[b, h, d]) * float(k[b, t, g, d]) for d in range(D)) for t in ts]
            mx = max(sc)
            w = [math.exp(x - mx) for x in sc]
            for d in range(D):
                want = sum(wi * float(v[b, t, g, d]) for wi, t in zip(w, ts)) / sum(w)
                assert abs(got[b, h, d] - want) < 1e-12
    k2, v2 = k.copy(), v.copy()
    k2[mask == 0] = 1e3
    v2[mask == 0] = -1e3
    assert oracle.dense_masked_decode(k2, v2, mask, q, "f32", 0.5).tobytes() == got.tobytes()


def check_validate_decode_inputs():
    """The oracle refuses inputs outside the decode's preconditions: a length
    past the table, a block outside the pool, a block shared by two logical
    blocks, query heads not a multiple of KV heads; well-formed inputs and
    padding entries (never read) pass."""
    tables = np.array([[3, 1, -7], [0, 2, 99]], np.int32)   # padding past ceil(T/B) ignored
    oracle.validate_decode_inputs(4, 4, tables, np.array([8, 6]), 8, 2)
    bad = [
        (np.array([[3, 1, -7], [0, 2, 99]], np.int32), np.array([13, 6]), 8, 2),   # 13 > 3*4
        (np.array([[3, 4, -7], [0, 2, 99]], np.int32), np.array([8, 6]), 8, 2),    # block 4 of 4
        (np.array([[3, 1, -7], [1, 2, 99]], np.int32), np.array([8, 6]), 8, 2),    # 1 twice
        (np.array([[3, 1, -7], [0, 2, 99]], np.int32), np.array([8, 6]), 6, 4),    # 6 % 4
        (np.array([[3, 1, -7], [0, 2, 99]], np.int32), np.array([-1, 6]), 8, 2),   # negative
    ]
    for t, lens, hq, hkv in bad:
        with pytest.raises(ValueError):
            oracle.validate_decode_inputs(4, 4, t, lens, hq, hkv)


def check_widen_f16():
    """Every finite binary16 pattern widens to the value its bits define;
    a few by hand: 1, -2, 0.25, the largest finite 65504, the smallest
    subnormal 2^-24 and -2^-14."""
    hand = np.array([0x3C00, 0xC000, 0x3400, 0x7BFF, 0x0001, 0x8400], np.uint16)
    assert oracle.widen(hand.view(np.float16), "f16").tolist() == \
        [1.0, -2.0, 0.25, 65504.0, 2.0 ** -24, -2.0 ** -14]
    bits = np.arange(1 << 16, dtype=np.uint32)
    finite = bits[((bits >> 10) & 0x1F) != 0x1F].astype(np.uint16)
    got = oracle.widen(finite.view(np.float16), "f16")
    want = np.array([_half_value_from_bits(int(u)) for u in finite])
    assert got.tobytes() == want.tobytes()


def check_widen():
    assert oracle.widen(np.array([0x3F80, 0xC000, 0x0000, 0x3E80], np.uint16), "bf16").tolist() == [1.0, -2.0, 0.0, 0.25]


ALL_CHECKS = [
    ("resolve_page_examples", check_resolve_page_examples),
    ("gather_coordinate_pool", check_gather_coordinate_pool),
    ("contiguous_equivalence_f32", lambda: check_contiguous_equivalence("f32")),
    ("contiguous_equivalence_bf16", lambda: check_contiguous_equivalence("bf16")),
    ("attention_vs_sdpa_f32", lambda: check_attention_vs_sdpa("f32")),
    ("attention_vs_sdpa_bf16", lambda: check_attention_vs_sdpa("bf16")),
    ("attention_vs_sdpa_f16", lambda: check_attention_vs_sdpa("f16")),
    ("contiguous_equivalence_f16", lambda: check_contiguous_equivalence("f16")),
    ("bruteforce_tiny", check_bruteforce_tiny),
    ("closed_forms", check_closed_forms),
    ("invariants", check_invariants),
    ("block_permutation_invariance", check_block_permutation_invariance),
    ("append_fixture", check_append_fixture),
    ("append_then_gather", check_append_then_gather),
    ("append_layers_fixture", check_append_layers_fixture),
    ("append_tokens_fixture", check_append_tokens_fixture),
    ("multi_appends_equal_single_appends", check_multi_appends_equal_single_appends),
    ("waste_examples", check_waste_examples),
    ("free_stack", check_free_stack),
    ("block_manager_page_figures", check_block_manager_page_figures),
    ("block_manager_lifo_reuse", check_block_manager_lifo_reuse),
    ("block_manager_admission", check_block_manager_admission),
    ("block_manager_random_invariants", check_block_manager_random_invariants),
    ("widen", check_widen),
    ("widen_f16", check_widen_f16),
    ("dense_masked_decode", check_dense_masked_decode),
    ("validate_decode_inputs", check_validate_decode_inputs),
]


@pytest.mark.parametrize("name,check", ALL_CHECKS, ids=[n for n, _ in ALL_CHECKS])
def test_pin(name, check):
    check()


# ----------------------------------------------------------------------------
# planted mistakes: every mutant must trip at least one pin
# ----------------------------------------------------------------------------

_orig_l2p = P.logical_to_physical
_orig_attend = P.attend
_orig_gather_seq = P.gather_sequence
_orig_widen = P.widen
_orig_dense = P.dense_masked_decode


def _mut_l2p_swapped(table_row, t, bs):
    return int(table_row[t % bs]), t // bs


def _mut_l2p_offby1(table_row, t, bs):
    return int(table_row[(t + 1) // bs]), (t + 1) % bs


def _mut_kv_head_modulo(h, hq, hkv):
    return h % hkv


def _attend_variant(*, scale_on=True, swap_kv=False, normalise=True, transpose_q=False):
    def f(q, K, V, scale):
        Hq, D = q.shape
        T, Hkv, _ = K.shape
        out = np.zeros((Hq, D))
        if T == 0:
            return out
        for h in range(Hq):
            g = P.kv_head_of(h, Hq, Hkv)
            KK, VV = (V, K) if swap_kv else (K, V)
            qq = q[h][::-1] if transpose_q else q[h]
            s = (scale if scale_on else 1.0) * (KK[:, g, :] @ qq)
            w = np.exp(s - s.max())
            out[h] = ((w / w.sum()) if normalise else w) @ VV[:, g, :]
        return out
    return f


def _mut_gather_layer0(pool, layer, table_row, T):
    return _orig_gather_seq(pool, 0, table_row, T)


def _mut_gather_kv_swapped(pool, layer, table_row, T):
    K, V = _orig_gather_seq(pool, layer, table_row, T)
    return V, K


def _mut_append_next_slot(pool, layer, block_tables, positions, k_new, v_new, *, in_place=False):
    out = pool if in_place else pool.copy()
    bs = pool.shape[4]
    for b in range(len(positions)):
        pos = int(positions[b]) + 1
        phys, off = _orig_l2p(block_tables[b], pos, bs)
        out[phys, 0, layer, :, off, :] = k_new[b]
        out[phys, 1, layer, :, off, :] = v_new[b]
    return out


_orig_append_tokens = P.kv_append_tokens


def _mut_append_tokens_shifted(pool, layer, block_tables, start_positions, token_offsets, k_new,
                               v_new, *, in_place=False):
    return _orig_append_tokens(pool, layer, block_tables, np.where(start_positions >= 0,
                               start_positions + 1, start_positions), token_offsets, k_new, v_new,
                               in_place=in_place)


def _mut_append_layers_first_only(pool, block_tables, positions, k_new, v_new, *, in_place=False):
    out = pool if in_place else pool.copy()
    P.kv_append(out, 0, block_tables, positions, k_new[:, 0], v_new[:, 0], in_place=True)
    return out


def _mut_waste_floor(n, bs):
    return (n // bs) * bs - n + bs - 1 if n % bs else 0


def _mut_widen_f16_as_bf16(x, dtype):
    if dtype == "f16":
        return _orig_widen(np.asarray(x).view(np.uint16), "bf16")
    return _orig_widen(x, dtype)


def _mut_dense_ignores_mask(k, v, mask, q, dtype, scale, seqs=None):
    return _orig_dense(k, v, np.ones_like(mask), q, dtype, scale, seqs)


def _mut_widen_low_half(x, dtype):
    if dtype == "bf16":
        return np.asarray(x, np.uint16).astype(np.float64)
    return np.asarray(x, np.float32).astype(np.float64)


MUTANTS = [
    ("l2p_swapped", "logical_to_physical", _mut_l2p_swapped),
    ("l2p_off_by_one", "logical_to_physical", _mut_l2p_offby1),
    ("kv_head_modulo", "kv_head_of", _mut_kv_head_modulo),
    ("attend_no_scale", "attend", _attend_variant(scale_on=False)),
    ("attend_swapped_kv", "attend", _attend_variant(swap_kv=True)),
    ("attend_unnormalised", "attend", _attend_variant(normalise=False)),
    ("attend_reversed_q", "attend", _attend_variant(transpose_q=True)),
    ("gather_ignores_layer", "gather_sequence", _mut_gather_layer0),
    ("gather_kv_swapped", "gather_sequence", _mut_gather_kv_swapped),
    ("append_next_slot", "kv_append", _mut_append_next_slot),
    ("append_tokens_shifted", "kv_append_tokens", _mut_append_tokens_shifted),
    ("append_layers_first_only", "kv_append_layers", _mut_append_layers_first_only),
    ("waste_floor", "paged_waste_slots", _mut_waste_floor),
    ("widen_low_half", "widen", _mut_widen_low_half),
    ("widen_f16_as_bf16", "widen", _mut_widen_f16_as_bf16),
    ("dense_ignores_mask", "dense_masked_decode", _mut_dense_ignores_mask),
]


_Model = oracle.BlockManagerModel
_orig_reserve = _Model.reserve


def _mut_blocks_floor_plus_one(self, n):
    return n // self.block_size + 1


def _mut_release_last_first(self, seq):
    for blk in reversed(self.tables.pop(seq)):
        self.stack.free(blk)
    del self.lens[seq]


def _mut_reserve_partial(self, seqs, counts):
    """allocates what it can before failing"""
    seqs, counts = list(seqs), list(counts)
    self._check_step(seqs, counts)
    starts = []
    for s, c in zip(seqs, counts):
        while len(self.tables[s]) < self.blocks_for(self.lens[s] + c):
            self.tables[s].append(self.stack.allocate())
        starts.append(self.lens[s])
        self.lens[s] += c
    return starts


def _mut_needed_ignores_full_tail(self, seqs, counts):
    return sum(self.blocks_for(c) for c in counts)


MANAGER_MUTANTS = [
    ("manager_blocks_floor_plus_one", "blocks_for", _mut_blocks_floor_plus_one),
    ("manager_release_last_first", "release", _mut_release_last_first),
    ("manager_reserve_partial", "reserve", _mut_reserve_partial),
    ("manager_needed_ignores_tail", "blocks_needed", _mut_needed_ignores_full_tail),
]


@pytest.mark.parametrize("name,attr,mutant", MANAGER_MUTANTS, ids=[m[0] for m in MANAGER_MUTANTS])
def test_manager_mutants_are_caught(name, attr, mutant):
    with mock.patch.object(_Model, attr, mutant):
        failed = []
        for cname, check in ALL_CHECKS:
            try:
                check()
            except (AssertionError, Exception):  # noqa: BLE001 - any failure counts
                failed.append(cname)
        assert failed, f"mutant {name} passed every pin"


@pytest.mark.parametrize("name,attr,mutant", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutants_are_caught(name, attr, mutant):
    patches = [mock.patch.object(P, attr, mutant)]
    # the package re-exports names; patch those too so checks see the mutant
    if hasattr(oracle, attr):
        patches.append(mock.patch.object(oracle, attr, mutant))
    for p in patches:
        p.start()
    try:
        failed = []
        for cname, check in ALL_CHECKS:
            try:
                check()
            except (AssertionError, Exception):  # noqa: BLE001 - any failure counts
                failed.append(cname)
        assert failed, f"mutant {name} passed every pin"
    finally:
        for p in reversed(patches):
            p.stop()
