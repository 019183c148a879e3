"""Paged-attention decode benchmark on one MI355X.

A step is one pass of the decode hot path over one batch, for one layer: each
sequence's new token K/V goes into its tail block and paged-attention decode
runs over the cache (block-table resolve, K/V stream, scaled QK^T, online
softmax, PV, split merge, output write), both in one library call
(paged_attention_decode_append, issued through a DecodePlan: the step's
buffers are fixed, so they are checked once).

    python bench.py [--workload llama8b_decode_bf16] [--steps K] [--warmup W]
                    [--extra long_context_bf16,churned_pool_bf16_gqa7]

Prints one JSON line.  The top level is the main workload (the Llama-8B-
shaped layer by default): `value` is effective HBM GB/s of its step
(algorithmic bytes / step time, inputs resident in HBM).  `workloads` holds
the same measurement for each --extra workload (by default the long-context
batch, the other configuration the 70%-of-peak target names, and the
churned-pool batch with its standalone one-token append).  Beside them: the
batched paged-KV gather and the dense decode over its output, the two
multi-row appends, the host block manager, an HBM read-ceiling probe, and
the CPU oracle's rate on a bounded sample.  Inputs are rotated among
replicas (same context lengths, redrawn tables and values) so that
consecutive steps do not hit in the 256 MB Infinity Cache.

    python bench.py --all-workloads --results-out profiles/results.json
    python bench.py --render profiles/results.json

measure every workload (one record each) and print the results table built
from such a record.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
MALL_BYTES = 256 << 20
ROOT = os.path.dirname(os.path.abspath(__file__))
PASS1_SOURCE = os.path.join(ROOT, "paged_kv_cache_resolve_amd", "csrc", "decode_mfma.hip")

# HBM bytes per decode pass-1 launch (the per-pair kernel where the step
# runs it), from two rocprofv3 PMC passes (FETCH_SIZE x 2.000 + WRITE_SIZE
# x 1.000; the factors make a 1 GiB device copy read and write 1 GiB),
# averaged over the dispatches of the profiled run (the input replicas share
# the context lengths, so they move the same bytes).  Only valid for the pass-1 kernel source whose SHA-256 is recorded;
# otherwise the JSON reports null.
MEASURED_TRAFFIC = {
    "llama8b_decode_bf16": {
        "kernel_sha256": "37b226c30e9e3ea4fc5d01075410df2a24e33e0dc619b2b2c6503a624b334a34",
        "bytes": 542140621,
    },
    "long_context_bf16": {
        "kernel_sha256": "37b226c30e9e3ea4fc5d01075410df2a24e33e0dc619b2b2c6503a624b334a34",
        "bytes": 2211046605,
    },
    "churned_pool_bf16_gqa7": {
        "kernel_sha256": "37b226c30e9e3ea4fc5d01075410df2a24e33e0dc619b2b2c6503a624b334a34",
        "bytes": 19310797,
    },
    "high_concurrency_bf16": {
        "kernel_sha256": "37b226c30e9e3ea4fc5d01075410df2a24e33e0dc619b2b2c6503a624b334a34",
        "bytes": 3819921408,
    },
    "tiny_fp32_mha": {
        "kernel_sha256": "37b226c30e9e3ea4fc5d01075410df2a24e33e0dc619b2b2c6503a624b334a34",
        "bytes": 620134,
    },
    "llama8b_decode_f32": {
        "kernel_sha256": "37b226c30e9e3ea4fc5d01075410df2a24e33e0dc619b2b2c6503a624b334a34",
        "bytes": 1146355098,
    },
    "llama8b_decode_f16": {
        "kernel_sha256": "37b226c30e9e3ea4fc5d01075410df2a24e33e0dc619b2b2c6503a624b334a34",
        "bytes": 582644326,
    },
    "gemma_like_d256_bf16": {
        "kernel_sha256": "37b226c30e9e3ea4fc5d01075410df2a24e33e0dc619b2b2c6503a624b334a34",
        "bytes": 1134821683,
    },
    "mqa32_decode_bf16": {
        "kernel_sha256": "37b226c30e9e3ea4fc5d01075410df2a24e33e0dc619b2b2c6503a624b334a34",
        "bytes": 87819162,
    },
    "mqa32_high_concurrency_bf16": {
        "kernel_sha256": "37b226c30e9e3ea4fc5d01075410df2a24e33e0dc619b2b2c6503a624b334a34",
        "bytes": 486555341,
    },
}

WORKLOADS = {
    "tiny_fp32_mha": 0,
    "churned_pool_bf16_gqa7": 1,
    "llama8b_decode_bf16": 2,
    "long_context_bf16": 3,
    "high_concurrency_bf16": 4,
    "llama8b_decode_f32": 5,
    "llama8b_decode_f16": 6,
    "gemma_like_d256_bf16": 7,
    "mqa32_decode_bf16": 8,
    "mqa32_high_concurrency_bf16": 9,
}


def pass1_source_sha() -> str:
    """SHA-256 of the pass-1 kernel source with comments and whitespace
    removed: the code the counters were taken on, not its commentary."""
    import hashlib
    import re
    with open(PASS1_SOURCE, encoding="utf-8") as f:
        src = f.read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    src = re.sub(r"\s+", "", src)
    return hashlib.sha256(src.encode()).hexdigest()


def measured_traffic(workload: str):
    rec = MEASURED_TRAFFIC.get(workload)
    if rec is None or rec["kernel_sha256"] != pass1_source_sha():
        return None
    return rec["bytes"]


def decode_bytes(w) -> int:
    """Algorithmic bytes of one decode: every cached K/V row once, q in, out
    out, the used block-table entries and the context lengths."""
    e = 4 if w.dtype == "f32" else 2
    T = w.context_lens.astype(np.int64)
    kv = int((2 * T * w.Hkv * w.D * e).sum())
    qo = w.S * w.Hq * w.D * 2 * e
    tables = 4 * int(((T + w.BS - 1) // w.BS).sum())
    return kv + qo + tables + 4 * w.S


def append_bytes(w) -> int:
    e = 4 if w.dtype == "f32" else 2
    return 2 * (2 * w.S * w.Hkv * w.D * e) + 4 * w.S + 4 * w.S


def gather_bytes(w, max_len: int) -> int:
    e = 4 if w.dtype == "f32" else 2
    T = w.context_lens.astype(np.int64)
    read = int((2 * T * w.Hkv * w.D * e).sum()) + 4 * int(((T + w.BS - 1) // w.BS).sum()) + 4 * w.S
    write = 2 * w.S * max_len * w.Hkv * w.D * e + w.S * max_len
    return read + write


def measure_appends(torch, pk, calls: int = 64) -> dict:
    """The two multi-row appends on Llama-8B KV geometry (8 KV heads,
    head_dim 128, block 16, bf16) in a 32-layer pool:

    - prompt: kv_append_tokens of 64 prompts x 512 tokens into one layer
      (rotating over the 32 layers and two input replicas, so neither the
      rows nor the destination stay in the 256 MB Infinity Cache);
    - decode: kv_append_layers of one token for 64 sequences in all 32
      layers, beside the same rows written by 32 kv_append calls.

    Algorithmic bytes: every new row read once and written once, plus the
    int32 tables, start positions and offsets."""
    S, T, L, Hkv, D, BS, e = 64, 512, 32, 8, 128, 16, 2
    mb = T // BS
    nb = S * mb
    gen = torch.Generator(device="cpu").manual_seed(77)
    pool_t = torch.empty(nb, 2, L, Hkv, BS, D, dtype=torch.bfloat16, device="cuda")
    pool = pk.KVPool(nb, BS, L, Hkv, D, torch.bfloat16, data=pool_t)
    tables = torch.randperm(nb, generator=gen).to(torch.int32).view(S, mb).cuda()
    rows = S * T
    reps = [(torch.randn(rows, Hkv, D, generator=gen).to(torch.bfloat16).cuda(),
             torch.randn(rows, Hkv, D, generator=gen).to(torch.bfloat16).cuda())
            for _ in range(2)]
    starts = torch.zeros(S, dtype=torch.int32, device="cuda")
    offsets = torch.arange(0, rows + 1, T, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()

    def timed(fn, n):
        fn(0)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for i in range(n):
            fn(i)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    def prompt(i):
        k, v = reps[i % 2]
        pk.kv_append_tokens(pool, (i // 2) % L, k, v, tables, starts, offsets)

    p_ms = timed(prompt, calls)
    p_bytes = 2 * 2 * rows * Hkv * D * e + 4 * S * mb + 4 * S + 4 * (S + 1)
    # the same bytes moved by a plain contiguous device copy (torch copy_), for scale
    dst = [torch.empty_like(reps[0][0]) for _ in range(2)]

    def plain_copy(i):
        k, v = reps[i % 2]
        dst[0].copy_(k)
        dst[1].copy_(v)

    c_ms = timed(plain_copy, calls)
    del dst

    kl = torch.randn(S, L, Hkv, D, generator=gen).to(torch.bfloat16).cuda()
    vl = torch.randn(S, L, Hkv, D, generator=gen).to(torch.bfloat16).cuda()
    pos = torch.randint(0, T, (S,), generator=gen).to(torch.int32).cuda()
    l_ms = timed(lambda i: pk.kv_append_layers(pool, kl, vl, tables, pos), calls)
    l_bytes = 2 * 2 * S * L * Hkv * D * e + 4 * S * 2
    ks = [kl[:, layer].contiguous() for layer in range(L)]
    vs = [vl[:, layer].contiguous() for layer in range(L)]

    def per_layer(i):
        for layer in range(L):
            pk.kv_append(pool, layer, ks[layer], vs[layer], tables, pos)

    s_ms = timed(per_layer, max(4, calls // 8))
    del pool, pool_t, reps
    return {
        "prompt_append": {
            "workload": "kv_append_tokens, 64 prompts x 512 tokens, 8 KV heads, head_dim 128, "
                        "block 16, bf16, 32-layer pool",
            "ms": round(p_ms, 5), "bytes": p_bytes,
            "GB_per_s": round(p_bytes / (p_ms * 1e-3) / 1e9, 1),
            "frac": round(p_bytes / (p_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "plain_copy_same_bytes_GB_per_s": round(p_bytes / (c_ms * 1e-3) / 1e9, 1)},
        "all_layer_append": {
            "workload": "kv_append_layers, 64 sequences x 32 layers, 8 KV heads, head_dim 128, "
                        "bf16",
            "ms": round(l_ms, 5), "bytes": l_bytes,
            "GB_per_s": round(l_bytes / (l_ms * 1e-3) / 1e9, 1),
            "ms_as_32_kv_append_calls": round(s_ms, 5)},
    }


def measure_manager(torch, pk, w, steps: int = 2000) -> dict:
    """Host cost of the block manager around one decode step of batch w:
    admission + tail allocation for one token per sequence
    (BlockManager.reserve) and the host block tables and lengths for the step
    (BlockManager.block_tables), through the Python binding."""
    bs = w.BS
    need = int(((w.context_lens.astype(np.int64) + steps + bs - 1) // bs).sum())
    pool = pk.KVPool(need, bs, 1, 1, 8, torch.bfloat16)   # tiny rows: only ids matter here
    mb = int((int(w.context_lens.max()) + steps + bs - 1) // bs)
    mgr = pk.BlockManager(pool, mb)
    ids = list(range(w.S))
    for i in ids:
        mgr.add_sequence(i)
    mgr.reserve(ids, (w.context_lens - 1).tolist())
    ones = [1] * w.S
    t0 = time.perf_counter()
    for _ in range(steps):
        mgr.reserve(ids, ones)
        mgr.block_tables(ids)
    dt = (time.perf_counter() - t0) / steps
    st = mgr.stats()
    mgr.close()
    del pool
    return {"us_per_step": round(dt * 1e6, 2), "batch": w.S, "steps": steps,
            "waste_ratio_after": round(st["waste_ratio"], 5),
            "waste_slots_after": st["waste_slots"]}


def cpu_baseline(w, budget_tokens: int, min_seconds: float = 10.0):
    """The oracle, as it stands, on a bounded sample of the same batch: whole
    sequences in a seeded order until `budget_tokens` cached tokens, run
    repeatedly until `min_seconds` of CPU work; the median run is reported.
    `cores` is the BLAS thread count its matrix products run on;
    `host_cores_allowed` the CPUs this process may use."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        blas_threads = 1
    order = np.random.default_rng(7).permutation(w.S)
    seqs, toks = [], 0
    for b in order:
        seqs.append(int(b))
        toks += int(w.context_lens[b])
        if toks >= budget_tokens:
            break
    runs = []
    while sum(runs) < min_seconds and len(runs) < 100:
        t0 = time.perf_counter()
        oracle.paged_attention_decode(w.pool, w.dtype, w.layer, w.block_tables, w.context_lens,
                                      w.q, w.scale, seqs=seqs)
        runs.append(time.perf_counter() - t0)
    dt = float(np.median(runs))
    e = 4 if w.dtype == "f32" else 2
    sample_bytes = sum(2 * int(w.context_lens[b]) * w.Hkv * w.D * e for b in seqs) + \
        len(seqs) * w.Hq * w.D * 2 * e
    # the same sample with BLAS held to one thread
    single = None
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            runs1 = []
            while sum(runs1) < min_seconds / 2 and len(runs1) < 50:
                t0 = time.perf_counter()
                oracle.paged_attention_decode(w.pool, w.dtype, w.layer, w.block_tables,
                                              w.context_lens, w.q, w.scale, seqs=seqs)
                runs1.append(time.perf_counter() - t0)
        d1 = float(np.median(runs1))
        single = {"value": round(sample_bytes / d1 / 1e9, 4), "unit": "GB/s", "cores": 1,
                  "seconds_per_run": round(d1, 3), "runs": len(runs1)}
    except Exception:  # noqa: BLE001 - threadpoolctl missing: report the main row only
        single = None
    return {
        "value": round(sample_bytes / dt / 1e9, 4),
        "unit": "GB/s",
        "cores": int(blas_threads),
        "host_cores_allowed": len(os.sched_getaffinity(0)),
        "kind": "oracle",
        "sample": f"{len(seqs)} of {w.S} sequences ({toks} cached tokens) of the same batch, "
                  f"fp64 numpy gather-then-attend, median of {len(runs)} runs "
                  f"({sum(runs):.1f} s of CPU work)",
        "tokens_per_s": round(len(seqs) / dt, 3),
        "seconds_per_run": round(dt, 3),
        "single_core": single,
    }


def _to_dev(torch, x, dtype):
    """float32 / float16 array or bf16 bit patterns -> device tensor."""
    if dtype in ("f32", "f16"):
        return torch.from_numpy(np.ascontiguousarray(x)).cuda()
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda().view(torch.bfloat16)


TORCH_DTYPES = {"f32": "float32", "bf16": "bfloat16", "f16": "float16"}


def load_replicas(torch, pk, name: str, rotate: int, split: str):
    """The workload's input replicas on the GPU, each with a DecodePlan of the
    fused step.  Replica r > 0 keeps replica 0's context lengths (the same
    bytes) and redraws tables, pool values, q and new rows."""
    from workloads import make_workload
    idx = WORKLOADS[name]
    w0 = make_workload(idx)
    kvb = decode_bytes(w0)
    n = rotate or max(1, min(4, math.ceil(4 * MALL_BYTES / max(kvb, 1))))
    ws = [w0] + [make_workload(idx, seed_offset=r, keep_lens=True) for r in range(1, n)]
    tdt = getattr(torch, TORCH_DTYPES[w0.dtype])
    reps = []
    for w in ws:
        pool = pk.KVPool(w.NB, w.BS, w.L, w.Hkv, w.D, tdt, data=_to_dev(torch, w.pool, w.dtype))
        r = dict(w=w, pool=pool, tables=torch.from_numpy(w.block_tables).cuda(),
                 lens=torch.from_numpy(w.context_lens).cuda(),
                 pos=torch.from_numpy(w.positions).cuda(), q=_to_dev(torch, w.q, w.dtype),
                 k=_to_dev(torch, w.k_new, w.dtype), v=_to_dev(torch, w.v_new, w.dtype),
                 out=torch.empty(w.S, w.Hq, w.D, dtype=tdt, device="cuda"))
        r["plan"] = pk.DecodePlan(r["out"], r["q"], r["pool"], w.layer, r["tables"], r["lens"],
                                  w.scale, r["k"], r["v"], r["pos"], split=split)
        reps.append(r)
    print(f"[bench] workload {name}: S={w0.S} Hq={w0.Hq} Hkv={w0.Hkv} D={w0.D} BS={w0.BS} "
          f"sum(T)={int(w0.context_lens.sum())} replicas={n}", file=sys.stderr, flush=True)
    return reps


def _events(torch):
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def back_to_back_ms(torch, fn, n: int) -> float:
    """Mean duration of fn(i), i < n, enqueued back to back on the current
    stream between one pair of HIP events (after one untimed call)."""
    stream = torch.cuda.current_stream()
    fn(0)
    torch.cuda.synchronize()
    a, b = _events(torch)
    a.record(stream)
    for i in range(n):
        fn(i)
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / n


def measure_step(torch, pk, name: str, steps: int, warmup: int, split: str, rotate: int = 0,
                 graph: bool = True):
    """Time the fused decode step of workload `name`.  Returns (record, replicas).

    - ms_per_step: wall clock over exactly `steps` steps after `warmup`
      untimed ones, bracketed by torch.cuda.synchronize();
    - call_ms: the same call back to back between one pair of HIP events on
      the launch stream (>= 100 calls): the roofline's kernel time;
    - per-call event pairs for the p10/p50/p90 spread (each pair adds a small
      gap, so these read slightly high);
    - graph_ms_per_step: 32 steps captured in one HIP graph, replayed."""
    reps = load_replicas(torch, pk, name, rotate, split)
    w0 = reps[0]["w"]
    stream = torch.cuda.current_stream()

    def step(i):
        reps[i % len(reps)]["plan"].run()

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = _events(torch)
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / steps
    gpu_ms_per_step = e0.elapsed_time(e1) / steps

    n_dec = max(steps, 100)
    call_ms = back_to_back_ms(torch, step, n_dec)
    ev = [_events(torch) for _ in range(n_dec)]
    for i in range(n_dec):
        ev[i][0].record(stream)
        step(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    per_call = [a.elapsed_time(b) for a, b in ev]

    graph_ms = None
    if graph:
        try:
            gplans = []
            for r in reps:
                w = r["w"]
                wsb = pk.paged_attention_workspace_bytes(r["pool"], w.S, w.Hq)
                gplans.append(pk.DecodePlan(
                    r["out"], r["q"], r["pool"], w.layer, r["tables"], r["lens"], w.scale,
                    r["k"], r["v"], r["pos"],
                    workspace=torch.zeros(wsb, dtype=torch.uint8, device="cuda"), split=split))
            n_graph = 32

            def graph_body():
                for i in range(n_graph):
                    gplans[i % len(gplans)].run()

            side = torch.cuda.Stream()
            side.wait_stream(stream)
            with torch.cuda.stream(side):
                graph_body()
            stream.wait_stream(side)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                graph_body()
            g.replay()
            torch.cuda.synchronize()
            g0, g1 = _events(torch)
            g0.record(stream)
            for _ in range(5):
                g.replay()
            g1.record(stream)
            torch.cuda.synchronize()
            graph_ms = g0.elapsed_time(g1) / (5 * n_graph)
            del g, gplans
        except RuntimeError as exc:   # capture unavailable: report it, keep the rest
            print(f"[bench] graph replay skipped: {exc}", file=sys.stderr, flush=True)

    # Which pass-1 form the call took: the chunk split's pass 1 writes the
    # per-sequence chunk prefix at the start of the workspace (its first
    # section), the per-pair kernel leaves it untouched.  The rest of the
    # workspace stays zero, as the library requires of a new workspace.  (One
    # more step on replica 0: it appends the same rows again, which leaves
    # the pool as it was.)
    r0 = reps[0]
    nbytes = pk.paged_attention_workspace_bytes(r0["pool"], w0.S, w0.Hq)
    probe = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    probe[: 4 * (w0.S + 1)] = 0xA5
    pk.paged_attention_decode_append(r0["out"], r0["q"], r0["pool"], w0.layer, r0["tables"],
                                     r0["lens"], w0.scale, r0["k"], r0["v"], r0["pos"],
                                     workspace=probe, split=split)
    torch.cuda.synchronize()
    split_used = "chunks" if bool((probe[: 4 * (w0.S + 1)] != 0xA5).any().item()) else "pairs"
    del probe

    step_bytes = float(np.mean([decode_bytes(r["w"]) + append_bytes(r["w"]) for r in reps]))
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    achieved = step_bytes / (call_ms * 1e-3) / 1e9
    rec = {
        "workload": name,
        "value": round(value, 2),
        "unit": "GB/s",
        "ms_per_step": round(ms_per_step, 5),
        "pct_of_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "tokens_per_s": round(w0.S / (ms_per_step * 1e-3), 1),
        "gpu_ms_per_step": round(gpu_ms_per_step, 5),
        "call_ms": round(call_ms, 5),
        "graph_ms_per_step": None if graph_ms is None else round(graph_ms, 5),
        "calls_timed": n_dec,
        "call_ms_per_call_events_p10_p50_p90": [
            round(float(np.percentile(per_call, q)), 5) for q in (10, 50, 90)],
        "split_used": split_used,
        "dtype": w0.dtype,
        "config": {
            "workload": name,
            "batch": w0.S, "q_heads": w0.Hq, "kv_heads": w0.Hkv, "head_dim": w0.D,
            "block_size": w0.BS, "layers_in_pool": w0.L, "layer": w0.layer,
            "sum_context_tokens": int(w0.context_lens.astype(np.int64).sum()),
            "max_context": int(w0.context_lens.max()),
            "input_replicas": len(reps),
            "replicas_share_context_lens": True,
            "split": split,
            "parallelism": "single GPU",
        },
        "roofline": {
            "kernel": ("paged_attention_decode_append (one call: decode pass 1 reading the new "
                       "rows, the merge of split sequences and the row store)"
                       if split_used == "chunks" else
                       "paged_attention_decode_append (one call: the per-pair kernel, which "
                       "streams, merges in its workgroup and stores the new rows)"),
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(name),
            "algorithmic_bytes_per_launch": int(step_bytes),
        },
    }
    return rec, reps


def measure_layer_rotation(torch, pk, reps, split: str, rounds: int = 8) -> dict:
    """The same fused step on replica 0's pool, attending each of its layers
    in turn back to back.  The replicas of a small workload fit in the 256 MB
    Infinity Cache together, so its step timings see K/V that stayed in the
    cache since the previous step; cycling over every layer of the pool (a
    model's other layers do the same between two uses of one layer) moves
    that many distinct K/V bytes."""
    r = reps[0]
    w = r["w"]
    plans = [pk.DecodePlan(r["out"], r["q"], r["pool"], layer, r["tables"], r["lens"], w.scale,
                           r["k"], r["v"], r["pos"], split=split) for layer in range(w.L)]
    n = rounds * w.L
    ms = back_to_back_ms(torch, lambda i: plans[i % w.L].run(), n)
    step_bytes = decode_bytes(w) + append_bytes(w)
    return {
        "what": f"the fused step attending layers 0..{w.L - 1} of one pool in turn, back to back",
        "layers": w.L,
        "distinct_kv_MB": round(w.L * (decode_bytes(w) + append_bytes(w)) / 1e6, 1),
        "call_ms": round(ms, 5),
        "GB_per_s": round(step_bytes / (ms * 1e-3) / 1e9, 1),
    }


def measure_append_only(torch, pk, reps, n: int = 200) -> dict:
    """kv_append of one new token per sequence on its own (one launch).
    `ms_host_loop`: back to back from Python (each call goes through the
    binding's checks, so a small append is bound by the host); `ms`: 16
    appends (rotating over the replicas) captured in one HIP graph and
    replayed, i.e. the GPU time per append."""
    w0 = reps[0]["w"]
    stream = torch.cuda.current_stream()

    def app(i):
        r = reps[i % len(reps)]
        pk.kv_append(r["pool"], r["w"].layer, r["k"], r["v"], r["tables"], r["pos"])

    host_ms = back_to_back_ms(torch, app, n)
    graph_ms = None
    try:
        n_graph = 16
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            for i in range(n_graph):
                app(i)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n_graph):
                app(i)
        g.replay()
        torch.cuda.synchronize()
        a, b = _events(torch)
        a.record(stream)
        for _ in range(10):
            g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        graph_ms = a.elapsed_time(b) / (10 * n_graph)
        del g
    except RuntimeError as exc:
        print(f"[bench] append graph skipped: {exc}", file=sys.stderr, flush=True)
    b = append_bytes(w0)
    ms = graph_ms if graph_ms is not None else host_ms
    return {"what": "kv_append of one token per sequence (all KV heads of the attended layer)",
            "ms": round(ms, 5), "ms_host_loop": round(host_ms, 5), "bytes": b,
            "GB_per_s": round(b / (ms * 1e-3) / 1e9, 2)}


def measure_decode_only(torch, pk, reps, split: str, n: int = 200) -> float:
    """paged_attention_decode alone (no append), back to back, through a
    plain DecodePlan per replica (tensors checked once, as for the step)."""
    plans = [pk.DecodePlan(r["out"], r["q"], r["pool"], r["w"].layer, r["tables"], r["lens"],
                           r["w"].scale, split=split) for r in reps]
    return round(back_to_back_ms(torch, lambda i: plans[i % len(plans)].run(), n), 5)


def measure_gather(torch, pk, rec_call_ms, r, tdt) -> dict:
    w = r["w"]
    max_len = w.max_len
    out = {}
    stream = torch.cuda.current_stream()
    outs = (torch.empty(w.S, max_len, w.Hkv, w.D, dtype=tdt, device="cuda"),
            torch.empty(w.S, max_len, w.Hkv, w.D, dtype=tdt, device="cuda"),
            torch.empty(w.S, max_len, dtype=torch.uint8, device="cuda"))
    gev = [_events(torch) for _ in range(5)]
    pk.paged_kv_gather(r["pool"], w.layer, r["tables"], r["lens"], max_len, out=outs)
    for a, b in gev:
        a.record(stream)
        pk.paged_kv_gather(r["pool"], w.layer, r["tables"], r["lens"], max_len, out=outs)
        b.record(stream)
    torch.cuda.synchronize()
    gms = float(np.mean([a.elapsed_time(b) for a, b in gev]))
    gb = gather_bytes(w, max_len)
    out["gather"] = {"ms": round(gms, 4), "bytes": gb, "GB_per_s": round(gb / (gms * 1e-3) / 1e9, 1)}
    if w.dtype != "f32":
        # the rest of the gather-then-attend path: dense decode over the
        # padded batch (every max_len row, padding included)
        dout = torch.empty_like(r["q"])
        pk.dense_attention_decode(dout, r["q"], outs[0], outs[1], outs[2], w.scale)
        for a, b in gev:
            a.record(stream)
            pk.dense_attention_decode(dout, r["q"], outs[0], outs[1], outs[2], w.scale)
            b.record(stream)
        torch.cuda.synchronize()
        dms = float(np.mean([a.elapsed_time(b) for a, b in gev]))
        e = 2
        db = 2 * w.S * max_len * w.Hkv * w.D * e + w.S * max_len + 2 * w.S * w.Hq * w.D * e
        out["gather_then_dense"] = {
            "dense_ms": round(dms, 4), "dense_bytes": db,
            "dense_GB_per_s": round(db / (dms * 1e-3) / 1e9, 1),
            "total_ms": round(gms + dms, 4), "total_bytes": gb + db,
            "paged_step_ms": round(rec_call_ms, 4),
            "total_over_paged": round((gms + dms) / rec_call_ms, 2),
        }
    del outs
    return out


PROBE_LIB = os.path.join(ROOT, "paged_kv_cache_resolve_amd", "libpagedkv_probe.so")


def read_ceiling(torch, buffer_gib: int = 4) -> dict:
    """HBM read ceiling of this GPU from the committed probe kernel
    (include/pagedkv_probe.h): a 4 GiB buffer (16x the Infinity Cache) read
    as 1 MiB slabs in order and as 4/8/32/64 KiB slabs in a random order,
    at 256..2048 workgroups; the best rate of each pattern, in GB/s.  Also
    what one workgroup (one CU) streams on its own, and each of eight
    (per_workgroup_random_2KiB, GB/s per workgroup), and a single 512 MiB
    read at 256 workgroups (random_32KiB_512MiB_256wg)."""
    import ctypes
    lib = ctypes.CDLL(PROBE_LIB)
    fn = lib.pagedkv_read_probe
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int64,
                   ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    nbytes = buffer_gib << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    stream = torch.cuda.current_stream()
    grids = (256, 512, 1024, 2048)
    sink = torch.empty(max(grids) * 256, dtype=torch.int32, device="cuda")
    gen = torch.Generator(device="cpu").manual_seed(5)
    res = {"unit": "GB/s", "buffer_GiB": buffer_gib, "kernel": "pagedkv_read_probe"}
    best_wg = {}
    for label, slab, order in (("sequential_1MiB", 1 << 20, "seq"), ("random_4KiB", 4 << 10, "rand"),
                               ("random_8KiB", 8 << 10, "rand"), ("random_32KiB", 32 << 10, "rand"),
                               ("random_64KiB", 64 << 10, "rand")):
        n = nbytes // slab
        ids = (torch.arange(n, dtype=torch.int32) if order == "seq"
               else torch.randperm(n, generator=gen).to(torch.int32)).cuda()
        best, best_g = 0.0, None
        for g in grids:
            def run(_i, g=g):
                rc = fn(buf.data_ptr(), nbytes, ids.data_ptr(), n, slab, g, sink.data_ptr(),
                        stream.cuda_stream)
                if rc != 0:
                    raise RuntimeError(f"pagedkv_read_probe returned {rc}")
            ms = back_to_back_ms(torch, run, 5)
            gbs = n * slab / (ms * 1e-3) / 1e9
            if gbs > best:
                best, best_g = gbs, g
        res[label] = round(best, 1)
        best_wg[label] = best_g
        del ids
    res["best_workgroups"] = best_wg
    # What one CU streams: 2 MiB of random 2 KiB slabs (one block's K or V
    # part at head_dim 64 in 16-bit types) read by one workgroup (4
    # wavefronts, 32 KiB in flight each), and by eight, per workgroup.
    slab, n = 2 << 10, 1024
    ids = torch.randperm(nbytes // slab, generator=gen)[:n].to(torch.int32).cuda()
    per_wg = {}
    for g in (1, 8):
        def run(_i, g=g):
            rc = fn(buf.data_ptr(), nbytes, ids.data_ptr(), n, slab, g, sink.data_ptr(),
                    stream.cuda_stream)
            if rc != 0:
                raise RuntimeError(f"pagedkv_read_probe returned {rc}")
        ms = back_to_back_ms(torch, run, 20)
        per_wg[str(g)] = round(n * slab / (ms * 1e-3) / 1e9 / g, 1)
    res["per_workgroup_random_2KiB"] = per_wg
    # A read of the Llama-shaped step's size in its launch shape: 512 MiB of
    # random 32 KiB slabs by 256 workgroups of 4 wavefronts (start-up and
    # tail included, as in one decode call).
    slab, n = 32 << 10, (512 << 20) // (32 << 10)
    ids = torch.randperm(nbytes // slab, generator=gen)[:n].to(torch.int32).cuda()

    def run(_i):
        rc = fn(buf.data_ptr(), nbytes, ids.data_ptr(), n, slab, 256, sink.data_ptr(),
                stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"pagedkv_read_probe returned {rc}")
    ms = back_to_back_ms(torch, run, 20)
    res["random_32KiB_512MiB_256wg"] = round(n * slab / (ms * 1e-3) / 1e9, 1)
    del buf, sink, ids
    return res


def _ceiling_for(ceiling: dict, w) -> tuple:
    """The random-slab ceiling whose slab matches the contiguous bytes of one
    block's K (or V) part in the attended layer: block_size x kv_heads x
    head_dim elements."""
    e = 4 if w.dtype == "f32" else 2
    run = w.BS * w.Hkv * w.D * e
    best = None
    for kib in (4, 8, 32, 64):
        if kib << 10 <= run:
            best = kib
    if best is None:
        best = 4
    key = f"random_{best}KiB"
    return key, ceiling.get(key)


def render_table(path: str) -> str:
    """Markdown results table from a record written by --results-out: per
    workload the step and call times, effective GB/s, the fraction of the
    8 TB/s nameplate and of the measured read ceiling for slabs of the
    workload's block size, and the split used."""
    sys.path.insert(0, ROOT)
    from workloads import make_workload
    with open(path) as f:
        rec = json.load(f)
    ceil = rec.get("read_ceiling") or {}
    rows = ["| Workload | Step (wall clock) | Call back to back | Step GB/s | % of 8 TB/s "
            "(step / call) | Call / read ceiling (slab) | Split | tokens/s (one layer) |",
            "|---|---|---|---|---|---|---|---|"]
    for name, r in rec["workloads"].items():
        frac_call = r["roofline"]["frac"] * 100
        key, val = _ceiling_for(ceil, make_workload(WORKLOADS[name], with_pool=False))
        cfrac = (f"{r['roofline']['achieved'] / val * 100:.1f}% ({key.split('_')[1]})"
                 if val else "-")
        rows.append(f"| {name} | {r['ms_per_step'] * 1e3:.1f} µs | {r['call_ms'] * 1e3:.1f} µs | "
                    f"{r['value']:.0f} | {r['pct_of_peak']:.1f}% / {frac_call:.1f}% | {cfrac} | "
                    f"{r['split_used']} | {r['tokens_per_s']:.2g} |")
    notes = []
    if ceil:
        notes.append("Read ceiling (pagedkv_read_probe, 4 GiB buffer): " + ", ".join(
            f"{k.replace('_', ' ')} {ceil[k]:.0f} GB/s" for k in
            ("sequential_1MiB", "random_4KiB", "random_8KiB", "random_32KiB", "random_64KiB")
            if k in ceil) + ".")
        r512 = ceil.get("random_32KiB_512MiB_256wg")
        if r512:
            notes.append(f"A 512 MiB read of random 32 KiB slabs by 256 workgroups (the Llama-shaped "
                         f"step's size and launch shape, start-up and tail included): {r512:.0f} GB/s.")
        pw = ceil.get("per_workgroup_random_2KiB")
        if pw:
            notes.append(f"One workgroup (one CU, 4 wavefronts with 32 KiB in flight each) streams "
                         f"{pw['1']:.0f} GB/s of random 2 KiB slabs; eight stream "
                         f"{pw['8']:.0f} GB/s each.")
    cpu = rec.get("cpu_baseline")
    if cpu:
        one = cpu.get("single_core") or {}
        notes.append(f"CPU oracle ({cpu.get('workload', '')}, {cpu['sample']}): {cpu['value']} GB/s with "
                     f"{cpu['cores']} BLAS threads ({cpu.get('host_cores_allowed', '?')} cores allowed)"
                     + (f", {one['value']} GB/s on 1 thread." if one else "."))
    app = rec["workloads"].get("churned_pool_bf16_gqa7", {}).get("append_only")
    if app:
        host = app.get("ms_host_loop")
        notes.append(f"churned_pool_bf16_gqa7 one-token kv_append on its own: {app['ms'] * 1e3:.2f} µs "
                     f"per append replayed from a HIP graph ({app['bytes']} bytes)" +
                     (f"; {host * 1e3:.2f} µs per call from a Python loop." if host else "."))
    return "\n".join(rows) + ("\n\n" + "\n".join(notes) if notes else "")


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="llama8b_decode_bf16", choices=sorted(WORKLOADS))
    ap.add_argument("--extra", default="long_context_bf16,churned_pool_bf16_gqa7",
                    help="comma-separated workloads also measured (sub-records), or 'none'")
    ap.add_argument("--extra-steps", type=int, default=100)
    ap.add_argument("--rotate", type=int, default=0, help="input replicas (0 = auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-gather", action="store_true")
    ap.add_argument("--no-appends", action="store_true")
    ap.add_argument("--no-read-ceiling", action="store_true")
    ap.add_argument("--cpu-budget-tokens", type=int, default=0)
    ap.add_argument("--split", choices=("auto", "chunks"), default="auto",
                    help="decode work split: auto (per-pair workgroups for small batches) or "
                         "chunks (always the persistent chunk split)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="also run a plain device copy of MIB MiB (counter calibration)")
    ap.add_argument("--all-workloads", action="store_true",
                    help="measure every workload (a record per workload) and nothing else")
    ap.add_argument("--results-out", default=None, help="with --all-workloads: write the record")
    ap.add_argument("--render", default=None, metavar="RECORD",
                    help="print the markdown results table of a --results-out record and exit")
    args = ap.parse_args(argv)

    if args.render:
        print(render_table(args.render))
        return 0
    if args.gpus != 1:
        print(f"bench.py: this path runs on one GPU only; --gpus {args.gpus} is not supported",
              file=sys.stderr, flush=True)
        return 2

    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr, flush=True)
        return 2

    sys.path.insert(0, ROOT)
    import paged_kv_cache_resolve_amd as pk

    if args.all_workloads:
        out = {"workloads": {}, "steps": args.steps, "warmup": args.warmup, "split": args.split,
               "device": torch.cuda.get_device_name(0)}
        for name in sorted(WORKLOADS, key=WORKLOADS.get):
            rec, reps = measure_step(torch, pk, name, args.steps, args.warmup, args.split,
                                     args.rotate, graph=False)
            if name == "churned_pool_bf16_gqa7":
                rec["append_only"] = measure_append_only(torch, pk, reps)
                rec["all_layers_rotated"] = measure_layer_rotation(torch, pk, reps, args.split)
            rec["decode_only_call_ms"] = measure_decode_only(torch, pk, reps, args.split)
            out["workloads"][name] = rec
            print(f"[bench] {name}: {rec['ms_per_step'] * 1e3:.1f} us/step, "
                  f"{rec['pct_of_peak']:.1f}% of 8 TB/s", file=sys.stderr, flush=True)
            del reps
            torch.cuda.empty_cache()
        if not args.no_read_ceiling:
            out["read_ceiling"] = read_ceiling(torch)
        if not args.no_cpu_baseline:
            from workloads import make_workload
            out["cpu_baseline"] = cpu_baseline(make_workload(WORKLOADS["llama8b_decode_bf16"]),
                                               args.cpu_budget_tokens or 600000)
            out["cpu_baseline"]["workload"] = "llama8b_decode_bf16"
        text = json.dumps(out)
        if args.results_out:
            with open(args.results_out, "w") as f:
                f.write(json.dumps(out, indent=1) + "\n")
        print(text, flush=True)
        return 0

    rec, reps = measure_step(torch, pk, args.workload, args.steps, args.warmup, args.split,
                             args.rotate)
    w0 = reps[0]["w"]
    tdt = getattr(torch, TORCH_DTYPES[w0.dtype])
    result = {
        "metric": "decode-attn effective HBM GB/s (% of peak) + tokens/s at batch×context",
        "value": rec["value"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": rec["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w0.dtype,
        "data": "synthetic (seeded N(0,1) K/V/q, seeded context lengths and block tables)",
        "config": rec["config"],
    }
    for key in ("pct_of_peak", "tokens_per_s", "gpu_ms_per_step", "call_ms", "graph_ms_per_step",
                "calls_timed", "call_ms_per_call_events_p10_p50_p90", "split_used", "roofline"):
        result[key] = rec[key]

    if not args.no_gather:
        try:
            result.update(measure_gather(torch, pk, rec["call_ms"], reps[0], tdt))
        except torch.cuda.OutOfMemoryError:
            result["gather"] = None
    del reps
    torch.cuda.empty_cache()

    extras = [] if args.extra in ("", "none") else [x for x in args.extra.split(",") if x]
    subs = {}
    for name in extras:
        if name == args.workload:
            continue
        if name not in WORKLOADS:
            raise SystemExit(f"unknown workload {name}")
        sub, sreps = measure_step(torch, pk, name, args.extra_steps, args.warmup, args.split,
                                  args.rotate, graph=False)
        sub.pop("dtype", None)
        if name == "churned_pool_bf16_gqa7":
            sub["append_only"] = measure_append_only(torch, pk, sreps)
            sub["all_layers_rotated"] = measure_layer_rotation(torch, pk, sreps, args.split)
            sub["decode_only_call_ms"] = measure_decode_only(torch, pk, sreps, args.split)
        subs[name] = sub
        del sreps
        torch.cuda.empty_cache()
    if subs:
        result["workloads"] = subs

    if not args.no_appends:
        try:
            result["appends"] = measure_appends(torch, pk)
        except torch.cuda.OutOfMemoryError:
            result["appends"] = None
        from workloads import make_workload
        result["host_block_manager"] = measure_manager(torch, pk, make_workload(
            WORKLOADS[args.workload], with_pool=False))

    if not args.no_read_ceiling:
        try:
            ceiling = read_ceiling(torch)
            result["roofline"]["read_ceiling"] = ceiling
            key, val = _ceiling_for(ceiling, w0)
            if val:
                result["roofline"]["frac_of_read_ceiling"] = {
                    "pattern": key, "frac": round(result["roofline"]["achieved"] / val, 4)}
            for name, sub in subs.items():
                from workloads import make_workload
                wk = make_workload(WORKLOADS[name], with_pool=False)
                key, val = _ceiling_for(ceiling, wk)
                if val:
                    sub["roofline"]["frac_of_read_ceiling"] = {
                        "pattern": key, "frac": round(sub["roofline"]["achieved"] / val, 4)}
        except (OSError, RuntimeError, torch.cuda.OutOfMemoryError) as exc:
            result["roofline"]["read_ceiling"] = None
            print(f"[bench] read ceiling skipped: {exc}", file=sys.stderr, flush=True)

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        result["copy_calibration_bytes"] = n
        del src, dst

    if not args.no_cpu_baseline:
        budget = args.cpu_budget_tokens or 600000
        result["cpu_baseline"] = cpu_baseline(w0, budget)

    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
