"""Paged-attention decode benchmark on one MI355X.

A step is one pass of the decode hot path over one batch, for one layer: each
sequence's new token K/V goes into its tail block and paged-attention decode
runs over the cache (block-table resolve, K/V stream, scaled QK^T, online
softmax, PV, split merge, output write), both in one library call
(paged_attention_decode_append, issued through a DecodePlan: the step's
buffers are fixed, so they are checked once).  The batched paged-KV gather is timed
separately and reported beside the step, and so are the two multi-row appends
(a prompt's tokens into one layer; one token into every layer).

    python bench.py [--workload llama8b_decode_bf16] [--steps K] [--warmup W]

Prints one JSON line.  `value` is effective HBM GB/s of the step (algorithmic
bytes / step time, inputs resident in HBM).  Inputs are rotated among
replicas so that consecutive steps do not hit in the 256 MB Infinity Cache.
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

# HBM bytes per decode pass-1 launch, from two rocprofv3 PMC passes
# (FETCH_SIZE x 2.000 + WRITE_SIZE x 1.000; the factors make a 1 GiB device
# copy read and write 1 GiB), averaged over the rotated input replicas.  Only
# valid for the pass-1 kernel source whose SHA-256 is recorded; otherwise the
# JSON reports null.
MEASURED_TRAFFIC = {
    "llama8b_decode_bf16": {
        "kernel_sha256": "57688c5d3de5a480caf4f41e978bb86684ba7544d319a202748939e5ff6b5fa1",
        "bytes": 585595523,
    },
    "long_context_bf16": {
        "kernel_sha256": "57688c5d3de5a480caf4f41e978bb86684ba7544d319a202748939e5ff6b5fa1",
        "bytes": 2210996659,
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
    repeatedly until `min_seconds` of CPU work; the median run is reported."""
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
        "kind": "oracle",
        "sample": f"{len(seqs)} of {w.S} sequences ({toks} cached tokens) of the same batch, "
                  f"fp64 numpy gather-then-attend, median of {len(runs)} runs "
                  f"({sum(runs):.1f} s of CPU work)",
        "tokens_per_s": round(len(seqs) / dt, 3),
        "seconds_per_run": round(dt, 3),
        "single_core": single,
    }


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="llama8b_decode_bf16", choices=sorted(WORKLOADS))
    ap.add_argument("--rotate", type=int, default=0, help="input replicas (0 = auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-gather", action="store_true")
    ap.add_argument("--no-appends", action="store_true")
    ap.add_argument("--cpu-budget-tokens", type=int, default=0)
    ap.add_argument("--split", choices=("auto", "chunks"), default="auto",
                    help="decode work split: auto (per-pair workgroups for small batches) or "
                         "chunks (always the persistent chunk split and merge kernel)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="also run a plain device copy of MIB MiB (counter calibration)")
    args = ap.parse_args(argv)

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
    from workloads import make_workload
    pk.set_split_mode(pk.SPLIT_AUTO if args.split == "auto" else pk.SPLIT_CHUNKS)

    idx = WORKLOADS[args.workload]
    w0 = make_workload(idx)
    kvb = decode_bytes(w0)
    reps = args.rotate or max(1, min(4, math.ceil(4 * MALL_BYTES / max(kvb, 1))))
    ws = [w0] + [make_workload(idx, seed_offset=r) for r in range(1, reps)]
    print(f"[bench] workload {args.workload}: S={w0.S} Hq={w0.Hq} Hkv={w0.Hkv} D={w0.D} "
          f"BS={w0.BS} sum(T)={int(w0.context_lens.sum())} replicas={reps}", file=sys.stderr,
          flush=True)

    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[w0.dtype]

    def dev(x):
        if w0.dtype in ("f32", "f16"):
            return torch.from_numpy(np.ascontiguousarray(x)).cuda()
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda().view(torch.bfloat16)

    reps_dev = []
    for w in ws:
        pool = pk.KVPool(w.NB, w.BS, w.L, w.Hkv, w.D, tdt, data=dev(w.pool))
        reps_dev.append(dict(
            w=w, pool=pool, tables=torch.from_numpy(w.block_tables).cuda(),
            lens=torch.from_numpy(w.context_lens).cuda(),
            pos=torch.from_numpy(w.positions).cuda(), q=dev(w.q), k=dev(w.k_new), v=dev(w.v_new),
            out=torch.empty(w.S, w.Hq, w.D, dtype=tdt, device="cuda")))
        r = reps_dev[-1]
        # the step's buffers are fixed, so a plan checks them once
        r["plan"] = pk.DecodePlan(r["out"], r["q"], r["pool"], w.layer, r["tables"], r["lens"],
                                  w.scale, r["k"], r["v"], r["pos"])
    stream = torch.cuda.current_stream()

    def step(i):
        reps_dev[i % len(reps_dev)]["plan"].run()

    def ev_pair():
        return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    # Timed region: exactly `steps` steps, nothing else enqueued in between.
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = ev_pair()
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    gpu_ms_per_step = e0.elapsed_time(e1) / args.steps

    # The same call back to back on the same stream, bracketed by one event
    # pair: the average call duration used for the roofline.
    n_dec = max(args.steps, 100)
    torch.cuda.synchronize()
    d0, d1 = ev_pair()
    d0.record(stream)
    for i in range(n_dec):
        step(i)
    d1.record(stream)
    torch.cuda.synchronize()
    dec_avg_ms = d0.elapsed_time(d1) / n_dec
    # Per-call distribution (an event pair per call adds its own gaps, so
    # these read slightly high).
    ev = [ev_pair() for _ in range(n_dec)]
    for i in range(n_dec):
        ev[i][0].record(stream)
        step(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    dec_ms = [a.elapsed_time(b) for a, b in ev]

    # The same step replayed from a HIP graph: 32 consecutive steps (what one
    # iteration of a 32-layer model enqueues) captured once, replayed.  Each
    # plan gets its own workspace, since a capture uses its own stream.
    graph_ms = None
    try:
        gplans = []
        for r in reps_dev:
            w = r["w"]
            wsb = pk.paged_attention_workspace_bytes(r["pool"], w.S, w.Hq)
            gplans.append(pk.DecodePlan(
                r["out"], r["q"], r["pool"], w.layer, r["tables"], r["lens"], w.scale,
                r["k"], r["v"], r["pos"],
                workspace=torch.empty(wsb, dtype=torch.uint8, device="cuda")))
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
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            graph_body()
        graph.replay()
        torch.cuda.synchronize()
        g0, g1 = ev_pair()
        g0.record(stream)
        for _ in range(5):
            graph.replay()
        g1.record(stream)
        torch.cuda.synchronize()
        graph_ms = g0.elapsed_time(g1) / (5 * n_graph)
        del graph, gplans
    except RuntimeError as exc:   # capture unavailable: report it, keep the rest
        print(f"[bench] graph replay skipped: {exc}", file=sys.stderr, flush=True)

    # Which pass-1 form the call took: the chunk split's pass 1 writes the
    # per-sequence chunk prefix at the start of the workspace, the per-pair
    # kernel leaves it untouched.  (One more step on replica 0: it appends the
    # same rows again, which leaves the pool as it was.)
    r0 = reps_dev[0]
    probe = torch.full((pk.paged_attention_workspace_bytes(r0["pool"], w0.S, w0.Hq),), 0xA5,
                       dtype=torch.uint8, device="cuda")
    pk.paged_attention_decode_append(r0["out"], r0["q"], r0["pool"], w0.layer, r0["tables"],
                                     r0["lens"], w0.scale, r0["k"], r0["v"], r0["pos"],
                                     workspace=probe)
    torch.cuda.synchronize()
    split_used = "chunks" if bool((probe[: 4 * (w0.S + 1)] != 0xA5).any().item()) else "pairs"
    del probe

    step_bytes = np.mean([decode_bytes(r["w"]) + append_bytes(r["w"]) for r in reps_dev])
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    achieved = step_bytes / (dec_avg_ms * 1e-3) / 1e9
    tokens_per_s = w0.S / (ms_per_step * 1e-3)

    result = {
        "metric": "decode-attn effective HBM GB/s (% of peak) + tokens/s at batch\u00d7context",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w0.dtype,
        "data": "synthetic (seeded N(0,1) K/V/q, seeded context lengths and block tables)",
        "config": {
            "workload": args.workload,
            "batch": w0.S, "q_heads": w0.Hq, "kv_heads": w0.Hkv, "head_dim": w0.D,
            "block_size": w0.BS, "layers_in_pool": w0.L, "layer": w0.layer,
            "sum_context_tokens": int(w0.context_lens.sum()),
            "max_context": int(w0.context_lens.max()),
            "input_replicas": reps,
            "split": args.split,
            "parallelism": "single GPU",
        },
        "pct_of_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "tokens_per_s": round(tokens_per_s, 1),
        "gpu_ms_per_step": round(gpu_ms_per_step, 5),
        "call_ms": round(dec_avg_ms, 5),
        "graph_ms_per_step": None if graph_ms is None else round(graph_ms, 5),
        "calls_timed": n_dec,
        "call_ms_per_call_events_p10_p50_p90": [
            round(float(np.percentile(dec_ms, q)), 5) for q in (10, 50, 90)],
        "split_used": split_used,
        "roofline": {
            "kernel": ("paged_attention_decode_append (decode pass 1 reading the new rows, "
                       "then the split merge that also stores them)") if split_used == "chunks" else
                      ("paged_attention_decode_append (one kernel: per-pair pass 1, the merge of "
                       "its pieces and the row store in the same workgroup)"),
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(args.workload),
            "algorithmic_bytes_per_launch": int(step_bytes),
        },
    }

    if not args.no_gather:
        r = reps_dev[0]
        w = r["w"]
        max_len = w.max_len
        try:
            outs = (torch.empty(w.S, max_len, w.Hkv, w.D, dtype=tdt, device="cuda"),
                    torch.empty(w.S, max_len, w.Hkv, w.D, dtype=tdt, device="cuda"),
                    torch.empty(w.S, max_len, dtype=torch.uint8, device="cuda"))
            gev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(5)]
            pk.paged_kv_gather(r["pool"], w.layer, r["tables"], r["lens"], max_len, out=outs)
            for a, b in gev:
                a.record(stream)
                pk.paged_kv_gather(r["pool"], w.layer, r["tables"], r["lens"], max_len, out=outs)
                b.record(stream)
            torch.cuda.synchronize()
            gms = float(np.mean([a.elapsed_time(b) for a, b in gev]))
            gb = gather_bytes(w, max_len)
            result["gather"] = {"ms": round(gms, 4), "bytes": gb,
                                "GB_per_s": round(gb / (gms * 1e-3) / 1e9, 1)}
            if w.dtype != "f32":
                # the rest of the gather-then-attend path: dense decode over
                # the padded batch (every max_len row, padding included)
                dout = torch.empty_like(r["q"])
                pk.dense_attention_decode(dout, r["q"], outs[0], outs[1], outs[2], w.scale)
                for a, b in gev:
                    a.record(stream)
                    pk.dense_attention_decode(dout, r["q"], outs[0], outs[1], outs[2], w.scale)
                    b.record(stream)
                torch.cuda.synchronize()
                dms = float(np.mean([a.elapsed_time(b) for a, b in gev]))
                e = 2
                db = (2 * w.S * max_len * w.Hkv * w.D * e + w.S * max_len
                      + 2 * w.S * w.Hq * w.D * e)
                result["gather_then_dense"] = {
                    "dense_ms": round(dms, 4), "dense_bytes": db,
                    "dense_GB_per_s": round(db / (dms * 1e-3) / 1e9, 1),
                    "total_ms": round(gms + dms, 4),
                    "total_bytes": gb + db,
                    "paged_step_ms": round(dec_avg_ms, 4),
                    "total_over_paged": round((gms + dms) / dec_avg_ms, 2),
                }
            del outs
        except torch.cuda.OutOfMemoryError:
            result["gather"] = None

    if not args.no_appends:
        try:
            result["appends"] = measure_appends(torch, pk)
        except torch.cuda.OutOfMemoryError:
            result["appends"] = None

    if not args.no_appends:
        result["host_block_manager"] = measure_manager(torch, pk, w0)

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
