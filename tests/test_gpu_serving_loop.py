"""A decode loop with no model around it: the C++ block manager admits
prompts and decode steps, kv_append_tokens writes the prompts, and every
step is one paged_attention_decode_append.  Beside it the oracle runs the
same loop with its own manager model, pool and decode.  After every step the
block tables, the whole pool (bit-exact) and the attention output (within
the bf16 tolerance) must agree.  Sequences finish and new ones reuse their
blocks; one prompt is refused for lack of blocks and must change nothing.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_resolve_amd as pk
from workloads import bf16_round_bits

from gpu_helpers import assert_attention_close, dev_to_np, np_to_dev, say

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU"),
]

NB, BS, L, HKV, HQ, D, MB, LAYER = 40, 16, 2, 2, 8, 128, 12, 1


def rows(rng, n, heads):
    return bf16_round_bits(rng.standard_normal((n, heads, D), dtype=np.float32))


def test_serving_loop_against_oracle():
    rng = np.random.default_rng(2024)
    pool = pk.kv_pool_create(NB, BS, L, HKV, D, torch.bfloat16)
    mgr = pk.BlockManager(pool, MB)
    model = oracle.BlockManagerModel(NB, BS, MB)
    ref_pool = np.zeros((NB, 2, L, HKV, BS, D), dtype=np.uint16)
    scale = D ** -0.5

    def prompt(seq_ids, lengths):
        for s in seq_ids:
            mgr.add_sequence(s)
            model.add_sequence(s)
        starts = mgr.reserve(seq_ids, lengths)
        assert starts.tolist() == model.reserve(seq_ids, lengths)
        tables, _ = mgr.block_tables(seq_ids)
        offsets = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
        k, v = rows(rng, int(offsets[-1]), HKV), rows(rng, int(offsets[-1]), HKV)
        pk.kv_append_tokens(pool, LAYER, np_to_dev(k, "bf16"), np_to_dev(v, "bf16"),
                            torch.from_numpy(tables).cuda(), torch.from_numpy(starts).cuda(),
                            torch.from_numpy(offsets).cuda())
        oracle.kv_append_tokens(ref_pool, LAYER, tables, starts, offsets, k, v, in_place=True)

    prompt([10, 11, 12], [20, 33, 1])
    live = [10, 11, 12]
    next_id = 13
    for step in range(40):
        say(f"serving loop step {step}, live {live}")
        if step == 8:
            mgr.release(11)
            model.release(11)
            live.remove(11)
            prompt([next_id], [50])                   # reuses 11's blocks, last one first
            live.append(next_id)
            next_id += 1
        if step == 20:
            # three full-width prompts need 36 blocks; about 30 are free
            big = [97, 98, 99]
            for s in big:
                mgr.add_sequence(s)
                model.add_sequence(s)
            before = (mgr.stats(), pool.num_free)
            assert mgr.blocks_needed(big, [MB * BS] * 3) == 3 * MB > pool.num_free
            with pytest.raises(pk.OutOfBlocksError):
                mgr.reserve(big, [MB * BS] * 3)
            with pytest.raises(MemoryError):
                model.reserve(big, [MB * BS] * 3)
            assert (mgr.stats(), pool.num_free) == before
            for s in big:
                mgr.release(s)
                model.release(s)
        if step == 30:
            mgr.release(10)
            model.release(10)
            live.remove(10)

        ones = [1] * len(live)
        assert mgr.blocks_needed(live, ones) == model.blocks_needed(live, ones)
        positions = mgr.reserve(live, ones)
        assert positions.tolist() == model.reserve(live, ones)
        tables, lens = mgr.block_tables(live)
        ref_tables, ref_lens = model.block_tables(live)
        assert tables.tobytes() == ref_tables.tobytes() and lens.tobytes() == ref_lens.tobytes()

        q = rows(rng, len(live), HQ)
        k, v = rows(rng, len(live), HKV), rows(rng, len(live), HKV)
        out = torch.empty(len(live), HQ, D, dtype=torch.bfloat16, device="cuda")
        pk.paged_attention_decode_append(out, np_to_dev(q, "bf16"), pool, LAYER,
                                         torch.from_numpy(tables).cuda(),
                                         torch.from_numpy(lens).cuda(), scale,
                                         np_to_dev(k, "bf16"), np_to_dev(v, "bf16"),
                                         torch.from_numpy(positions).cuda())
        torch.cuda.synchronize()
        oracle.kv_append(ref_pool, LAYER, ref_tables, positions, k, v, in_place=True)
        ref = oracle.paged_attention_decode(ref_pool, "bf16", LAYER, ref_tables, ref_lens, q,
                                            scale)
        assert_attention_close(out, ref, "bf16", what=f"step {step}")
        assert dev_to_np(pool.data).tobytes() == ref_pool.tobytes(), f"pool differs at step {step}"
        assert mgr.stats() == model.stats()
    st = mgr.stats()
    assert st["waste_slots"] <= (BS - 1) * st["sequences"]
