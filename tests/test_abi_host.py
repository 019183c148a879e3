"""CPU-side checks of the C ABI: the library loads, exports every function
include/pagedkv.h declares, and its host logic (pool geometry, free-block
stack, argument validation) behaves as documented.  No GPU work is issued:
the pool handles here describe a fake device address that is never touched.
"""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from conftest import ROOT

import paged_kv_cache_resolve_amd as pk
from paged_kv_cache_resolve_amd import _lib

L = pk.library()
FAKE_DEVICE_PTR = ctypes.c_void_p(0x7F0000000000)


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "pagedkv.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\**\s+\**([a-z_][a-z0-9_]*)\s*\(",
                       text, flags=re.M)
    return sorted(set(names))


def test_every_declared_symbol_is_exported():
    names = _declared_functions()
    assert len(names) == 27, names
    for n in names:
        assert hasattr(L, n), f"{n} missing from libpagedkv.so"
    assert set(names) == set(_lib.SIGNATURES), "binding signatures drift from the header"


def test_decode_flags_are_per_call():
    """The decode split is a per-call flag: the only process-wide setter is
    gone, and a flag bit the header does not define is an argument error
    (host only, nothing enqueued)."""
    assert not hasattr(L, "paged_attention_set_split_mode")
    h = _pool(nb=8, layers=1, hkv=2, d=64)
    p = FAKE_DEVICE_PTR
    wsb = L.paged_attention_workspace_bytes(h, 4, 8)
    for bad in (2, 4, 0x80000000, 3):
        assert L.paged_attention_decode(p, p, h, 0, p, 4, p, 4, 8, ctypes.c_float(0.1), p, wsb,
                                        bad, None) == _lib.ERR_INVALID_ARG
        assert L.paged_attention_decode_append(p, p, p, p, p, h, 0, p, 4, p, 4, 8,
                                               ctypes.c_float(0.1), p, wsb, bad,
                                               None) == _lib.ERR_INVALID_ARG
    for ok in (0, _lib.DECODE_CHUNKS):   # batch 0: validated, nothing to do
        assert L.paged_attention_decode(p, p, h, 0, p, 4, p, 0, 8, ctypes.c_float(0.1), p, wsb,
                                        ok, None) == 0
    L.kv_pool_destroy(h)


def _pool(nb=10, bs=16, layers=2, hkv=2, d=64, dtype=_lib.BF16):
    h = ctypes.c_void_p()
    nbytes = L.kv_pool_bytes(nb, bs, layers, hkv, d, dtype)
    rc = L.kv_pool_create(ctypes.byref(h), nb, bs, layers, hkv, d, dtype, FAKE_DEVICE_PTR, nbytes)
    assert rc == 0
    return h


def test_pool_bytes():
    # the mini-infer pool defaults: 16 tokens x 24 layers x 2 heads x 64 dims, K and V, bf16
    assert L.kv_pool_bytes(1, 16, 24, 2, 64, _lib.BF16) == 196608
    assert L.kv_pool_bytes(3, 16, 1, 8, 128, _lib.F32) == 3 * 2 * 8 * 16 * 128 * 4
    assert L.kv_pool_bytes(0, 16, 1, 1, 8, _lib.BF16) == 0
    assert L.kv_pool_bytes(1, 16, 1, 1, 8, 7) == 0


def test_pool_create_validation():
    h = ctypes.c_void_p()
    need = L.kv_pool_bytes(4, 16, 1, 2, 64, _lib.BF16)
    assert L.kv_pool_create(ctypes.byref(h), 4, 16, 1, 2, 64, _lib.BF16, FAKE_DEVICE_PTR, need - 1) == -1
    assert L.kv_pool_create(ctypes.byref(h), 4, 16, 1, 2, 64, _lib.BF16, None, need) == -1
    assert L.kv_pool_create(ctypes.byref(h), 4, 16, 1, 2, 60, _lib.BF16, FAKE_DEVICE_PTR, need) == -1
    assert L.kv_pool_create(ctypes.byref(h), 4, 16, 1, 2, 64, _lib.BF16,
                            ctypes.c_void_p(0x7F0000000008), need) == -1
    assert L.kv_pool_create(None, 4, 16, 1, 2, 64, _lib.BF16, FAKE_DEVICE_PTR, need) == -1


def test_geometry_roundtrip():
    h = _pool(nb=7, bs=32, layers=3, hkv=4, d=128, dtype=_lib.F32)
    vals = [ctypes.c_int() for _ in range(6)]
    base = ctypes.c_void_p()
    assert L.kv_pool_geometry(h, *[ctypes.byref(v) for v in vals], ctypes.byref(base)) == 0
    assert [v.value for v in vals] == [7, 32, 3, 4, 128, _lib.F32]
    assert base.value == FAKE_DEVICE_PTR.value
    L.kv_pool_destroy(h)


def test_free_stack_matches_oracle_model():
    """Random allocate/free traffic: the library hands out exactly the ids the
    page's LIFO stack model hands out."""
    rng = np.random.default_rng(5)
    nb = 64
    h = _pool(nb=nb)
    model = oracle.FreeBlockStack(nb)
    held = []
    out = ctypes.c_int32()
    for _ in range(5000):
        if held and (rng.random() < 0.45 or len(model) == 0):
            i = int(rng.integers(len(held)))
            bid = held.pop(i)
            assert L.kv_pool_free_block(h, bid) == 0
            model.free(bid)
        else:
            rc = L.kv_pool_alloc_block(h, ctypes.byref(out))
            if len(model) == 0:
                assert rc == _lib.ERR_OUT_OF_BLOCKS
                with pytest.raises(MemoryError):
                    model.allocate()
                continue
            assert rc == 0
            assert out.value == model.allocate()
            held.append(out.value)
        assert L.kv_pool_num_free(h) == len(model)
    L.kv_pool_destroy(h)


def test_first_allocation_and_exhaustion():
    h = _pool(nb=3)
    out = ctypes.c_int32()
    got = []
    for _ in range(3):
        assert L.kv_pool_alloc_block(h, ctypes.byref(out)) == 0
        got.append(out.value)
    assert got == [2, 1, 0]
    assert L.kv_pool_alloc_block(h, ctypes.byref(out)) == _lib.ERR_OUT_OF_BLOCKS
    assert L.pagedkv_status_string(_lib.ERR_OUT_OF_BLOCKS) == b"no free block left in the pool"
    L.kv_pool_destroy(h)


def test_free_rejects_bad_ids():
    h = _pool(nb=4)
    out = ctypes.c_int32()
    assert L.kv_pool_free_block(h, 3) == _lib.ERR_INVALID_ARG     # already free
    assert L.kv_pool_free_block(h, 4) == _lib.ERR_INVALID_ARG     # out of range
    assert L.kv_pool_free_block(h, -1) == _lib.ERR_INVALID_ARG
    assert L.kv_pool_alloc_block(h, ctypes.byref(out)) == 0
    assert L.kv_pool_free_block(h, out.value) == 0
    assert L.kv_pool_free_block(h, out.value) == _lib.ERR_INVALID_ARG   # double free
    L.kv_pool_destroy(h)


def test_entry_points_validate_before_launch():
    """Host-checkable mistakes are rejected without touching the GPU."""
    h = _pool(nb=8, layers=2, hkv=2, d=64)
    p = FAKE_DEVICE_PTR
    ws_bytes = L.paged_attention_workspace_bytes(h, 4, 8)
    assert ws_bytes > 0
    assert L.paged_attention_workspace_bytes(h, 4, 7) == 0          # 7 % 2 != 0
    dec = lambda **kw: L.paged_attention_decode(  # noqa: E731
        kw.get("out", p), kw.get("q", p), h, kw.get("layer", 0), p, kw.get("mb", 4), p,
        kw.get("batch", 4), kw.get("hq", 8), ctypes.c_float(kw.get("scale", 0.125)),
        kw.get("ws", p), kw.get("wsb", ws_bytes), kw.get("flags", 0), None)
    assert dec(layer=2) == _lib.ERR_INVALID_ARG
    assert dec(layer=-1) == _lib.ERR_INVALID_ARG
    assert dec(hq=6 + 1) == _lib.ERR_INVALID_ARG
    assert dec(mb=0) == _lib.ERR_INVALID_ARG
    assert dec(batch=-1) == _lib.ERR_INVALID_ARG
    assert dec(out=None) == _lib.ERR_INVALID_ARG
    assert dec(scale=float("nan")) == _lib.ERR_INVALID_ARG
    ws34 = L.paged_attention_workspace_bytes(h, 4, 2 * 17)             # 17 heads per KV head
    assert ws34 > 0 and dec(hq=2 * 17, wsb=ws34 - 1) == _lib.ERR_WORKSPACE
    assert dec(wsb=ws_bytes - 1) == _lib.ERR_WORKSPACE
    assert dec(ws=None) == _lib.ERR_WORKSPACE
    assert dec(ws=ctypes.c_void_p(p.value + 64)) == _lib.ERR_WORKSPACE  # misaligned
    assert dec(batch=0) == 0                                            # nothing to do
    fused = lambda **kw: L.paged_attention_decode_append(  # noqa: E731
        p, p, kw.get("k", p), kw.get("v", p), kw.get("pos", p), h, kw.get("layer", 0), p, 4, p,
        kw.get("batch", 4), 8, ctypes.c_float(0.125), p, kw.get("wsb", ws_bytes), 0, None)
    assert fused(k=None) == _lib.ERR_INVALID_ARG
    assert fused(v=None) == _lib.ERR_INVALID_ARG
    assert fused(pos=None) == _lib.ERR_INVALID_ARG
    assert fused(layer=2) == _lib.ERR_INVALID_ARG
    assert fused(wsb=ws_bytes - 1) == _lib.ERR_WORKSPACE
    assert fused(batch=0, k=None, v=None, pos=None) == 0
    assert L.kv_append(h, 2, p, p, p, 4, p, 4, None) == _lib.ERR_INVALID_ARG
    assert L.kv_append(h, 0, None, p, p, 4, p, 4, None) == _lib.ERR_INVALID_ARG
    assert L.kv_append(h, 0, p, p, p, 4, p, 0, None) == 0
    assert L.paged_kv_gather(p, p, p, h, 5, p, 4, p, 4, 16, None) == _lib.ERR_INVALID_ARG
    assert L.paged_kv_gather(None, p, p, h, 0, p, 4, p, 4, 16, None) == _lib.ERR_INVALID_ARG
    assert L.paged_kv_gather(p, p, p, h, 0, p, 4, p, 4, 0, None) == 0
    odd = ctypes.c_void_p(p.value + 8)                                  # not 16-byte aligned
    assert dec(q=odd) == _lib.ERR_INVALID_ARG
    assert dec(out=odd) == _lib.ERR_INVALID_ARG
    assert fused(k=odd) == _lib.ERR_INVALID_ARG
    assert L.kv_append(h, 0, odd, p, p, 4, p, 4, None) == _lib.ERR_INVALID_ARG
    assert L.paged_kv_gather(p, odd, p, h, 0, p, 4, p, 4, 16, None) == _lib.ERR_INVALID_ARG
    # all-layer append: kv_append_layers(pool, k, v, tables, mb, positions, batch, stream)
    assert L.kv_append_layers(h, None, p, p, 4, p, 4, None) == _lib.ERR_INVALID_ARG
    assert L.kv_append_layers(h, p, p, p, 0, p, 4, None) == _lib.ERR_INVALID_ARG
    assert L.kv_append_layers(h, p, p, p, 4, p, -1, None) == _lib.ERR_INVALID_ARG
    assert L.kv_append_layers(h, p, odd, p, 4, p, 4, None) == _lib.ERR_INVALID_ARG
    assert L.kv_append_layers(h, None, None, None, 4, None, 0, None) == 0
    # multi-token append: kv_append_tokens(pool, layer, k, v, tables, mb, starts,
    #                                      offsets, batch, total, stream)
    tok = lambda **kw: L.kv_append_tokens(  # noqa: E731
        h, kw.get("layer", 0), kw.get("k", p), p, p, kw.get("mb", 4), p, kw.get("off", p),
        kw.get("batch", 4), kw.get("total", 40), None)
    assert tok(layer=2) == _lib.ERR_INVALID_ARG
    assert tok(mb=0) == _lib.ERR_INVALID_ARG
    assert tok(total=-1) == _lib.ERR_INVALID_ARG
    assert tok(batch=-1) == _lib.ERR_INVALID_ARG
    assert tok(off=None) == _lib.ERR_INVALID_ARG
    assert tok(k=odd) == _lib.ERR_INVALID_ARG
    assert tok(total=0, k=None, off=None) == 0
    assert tok(batch=0, k=None, off=None) == 0
    # dense decode: (out, q, k, v, mask, batch, max_len, kv_heads, head_dim, hq, dtype, scale, ws, wsb, stream)
    dws = L.dense_attention_workspace_bytes(4, 2, 8, 128)
    assert dws > 0 and L.dense_attention_workspace_bytes(4, 2, 7, 128) == 0
    dd = lambda **kw: L.dense_attention_decode(  # noqa: E731
        kw.get("out", p), p, kw.get("k", p), p, kw.get("mask", p), kw.get("batch", 4),
        kw.get("max_len", 40), 2, kw.get("d", 128), kw.get("hq", 8), kw.get("dtype", _lib.BF16),
        ctypes.c_float(0.1), kw.get("ws", p), kw.get("wsb", dws), None)
    assert dd(hq=7) == _lib.ERR_INVALID_ARG
    assert dd(mask=None) == _lib.ERR_INVALID_ARG
    assert dd(k=odd) == _lib.ERR_INVALID_ARG
    assert dd(max_len=-1) == _lib.ERR_INVALID_ARG
    assert dd(dtype=_lib.F32) == _lib.ERR_UNSUPPORTED
    assert dd(d=80) == _lib.ERR_UNSUPPORTED
    dws34 = L.dense_attention_workspace_bytes(4, 2, 2 * 17, 128)
    assert dws34 > 0 and dd(hq=2 * 17, wsb=dws34 - 1) == _lib.ERR_WORKSPACE
    assert dd(wsb=dws - 1) == _lib.ERR_WORKSPACE
    assert dd(batch=0, out=None) == 0
    assert L.paged_kv_resolve(p, p, 4, p, 4, 0, 16, None) == _lib.ERR_INVALID_ARG
    assert L.paged_kv_resolve(None, p, 4, p, 4, 16, 16, None) == _lib.ERR_INVALID_ARG
    L.kv_pool_destroy(h)


def _align256(n):
    return (n + 255) // 256 * 256


def _ws_bytes(batch, vheads, share, d):
    slots = batch * vheads + 8192
    return (_align256(4 * (batch + 1)) + _align256(4 * slots * share * 2) +
            _align256(4 * slots * share * d))


@pytest.mark.parametrize("hkv,hq,d,bs,dtype,qsplit,share", [
    (2, 8, 64, 16, _lib.BF16, 1, 4),
    (2, 32, 64, 16, _lib.BF16, 1, 16),
    (1, 32, 64, 16, _lib.BF16, 1, 32),     # MQA-32: one wavefront, two column groups
    (2, 34, 64, 16, _lib.BF16, 1, 17),
    (1, 48, 128, 16, _lib.F16, 2, 24),
    (1, 64, 64, 32, _lib.BF16, 2, 32),
    (1, 71, 64, 16, _lib.BF16, 3, 24),
    (1, 51, 128, 16, _lib.BF16, 2, 26),
    (1, 32, 96, 16, _lib.BF16, 2, 16),     # head_dim 96: 16 query heads per wavefront
    (1, 32, 64, 16, _lib.F32, 2, 16),      # fp32 stream: 16
    (1, 32, 64, 8, _lib.BF16, 2, 16),      # 8-token blocks: 16
    (1, 71, 256, 16, _lib.BF16, 5, 15),
    (2, 40, 80, 16, _lib.BF16, 2, 10),     # VALU kernel (head_dim 80): 16
])
def test_wide_groups_workspace(hkv, hq, d, bs, dtype, qsplit, share):
    """More query heads per KV head than one wavefront serves: the KV head is
    served as qsplit = ceil(G / W) virtual heads of at most share =
    ceil(G / qsplit) query heads, W = 32 for the 16-bit MFMA stream at
    head_dim 64 or 128 with blocks of a multiple of 16 tokens, else 16.  The
    workspace holds one partial slot per virtual head, `share` heads wide.
    The dense decode always splits at 16."""
    h = _pool(nb=8, bs=bs, layers=1, hkv=hkv, d=d, dtype=dtype)
    batch = 5
    assert L.paged_attention_workspace_bytes(h, batch, hq) == _ws_bytes(batch, hkv * qsplit, share, d)
    g = hq // hkv
    dq = -(-g // 16)
    assert L.dense_attention_workspace_bytes(batch, hkv, hq, d) == \
        _ws_bytes(batch, hkv * dq, -(-g // dq), d)
    L.kv_pool_destroy(h)


def test_binding_workspace_size_follows_pool_shape():
    """The binding asks the library for every workspace size: pools of the
    same head shape but another dtype or block size split their query heads
    differently (32 per wavefront only for 16-bit pools with blocks of a
    multiple of 16 tokens), so their sizes differ, whichever was asked first.
    A new pool that reuses a destroyed pool's handle address gets its own
    size too."""
    import types
    cases = [(1, 128, 16, _lib.F32), (1, 128, 16, _lib.BF16), (1, 64, 8, _lib.BF16),
             (1, 64, 16, _lib.BF16), (8, 128, 16, _lib.BF16), (2, 64, 16, _lib.F16)]
    sizes = []
    for hkv, d, bs, dt in cases:
        h = _pool(nb=8, bs=bs, layers=1, hkv=hkv, d=d, dtype=dt)
        pool = types.SimpleNamespace(handle=h, kv_heads=hkv, head_dim=d, block_size=bs, dtype=dt)
        got = pk.paged_attention_workspace_bytes(pool, 300, 32)
        assert got == L.paged_attention_workspace_bytes(h, 300, 32)
        sizes.append(got)
        L.kv_pool_destroy(h)
    # fp32 and 8-token blocks: 16 query heads per virtual head; bf16 with 16-token blocks: 32
    assert sizes[0] != sizes[1] and sizes[2] != sizes[3]


def test_decode_refuses_chunk_counts_past_int32():
    """The kernels keep per-sequence chunk counts and their prefix sums in
    int32: a batch whose tables allow more than 2^31 - 1 chunks of 16 tokens
    in total is refused before any launch."""
    h = _pool(nb=8, bs=16, layers=1, hkv=2, d=64)
    p = FAKE_DEVICE_PTR
    batch = 16384
    wsb = L.paged_attention_workspace_bytes(h, batch, 8)
    dec = lambda mb: L.paged_attention_decode(  # noqa: E731
        p, p, h, 0, p, mb, p, batch, 8, ctypes.c_float(0.1), p, wsb, 0, None)
    limit_mb = (2**31 - 1) // batch          # chunks per sequence that still fit
    assert dec(limit_mb + 1) == _lib.ERR_UNSUPPORTED
    assert dec(2**30) == _lib.ERR_UNSUPPORTED
    fused = L.paged_attention_decode_append(p, p, p, p, p, h, 0, p, limit_mb + 1, p, batch, 8,
                                            ctypes.c_float(0.1), p, wsb, 0, None)
    assert fused == _lib.ERR_UNSUPPORTED
    L.kv_pool_destroy(h)


def test_noalloc_decode_validates_and_refuses_oversized_calls():
    """paged_attention_decode_noalloc checks its arguments as
    paged_attention_decode does, and refuses a call whose workspace would
    exceed its 64 MiB static scratch with PAGEDKV_ERR_SCRATCH; both before
    anything touches the GPU."""
    h = _pool(nb=8, bs=16, layers=1, hkv=8, d=128)
    p = FAKE_DEVICE_PTR
    dec = lambda batch, hq=32, layer=0, flags=0, out=p: L.paged_attention_decode_noalloc(  # noqa: E731
        out, p, h, layer, p, 4, p, batch, hq, ctypes.c_float(0.1), flags, None)
    assert dec(4, layer=1) == _lib.ERR_INVALID_ARG
    assert dec(4, hq=31) == _lib.ERR_INVALID_ARG
    assert dec(4, flags=2) == _lib.ERR_INVALID_ARG
    assert dec(4, out=None) == _lib.ERR_INVALID_ARG
    assert dec(0) == 0
    assert dec(16385) == _lib.ERR_UNSUPPORTED
    limit = 64 << 20
    fits = [b for b in (1000, 2000, 3000, 4000, 8000, 16384)
            if L.paged_attention_workspace_bytes(h, b, 32) <= limit]
    over = [b for b in (1000, 2000, 3000, 4000, 8000, 16384)
            if L.paged_attention_workspace_bytes(h, b, 32) > limit]
    assert fits and over
    for b in over:
        assert dec(b) == _lib.ERR_SCRATCH
    assert b"64 MiB" in L.pagedkv_status_string(_lib.ERR_SCRATCH)
    L.kv_pool_destroy(h)


def test_build_module_runs_without_the_library(tmp_path):
    """`python -m paged_kv_cache_resolve_amd.build` works on a checkout where
    the library has not been built yet: importing the package does not load
    it, and the build writes it.  Run on a copy of the sources."""
    import shutil
    import subprocess
    import sys
    pkg = os.path.join(ROOT, "paged_kv_cache_resolve_amd")
    shutil.copytree(pkg, tmp_path / "paged_kv_cache_resolve_amd",
                    ignore=shutil.ignore_patterns("*.so", "*.so.tmp*", "_build", "__pycache__"))
    shutil.copytree(os.path.join(ROOT, "include"), tmp_path / "include")
    assert not (tmp_path / "paged_kv_cache_resolve_amd" / "libpagedkv.so").exists()
    env = dict(os.environ)
    env.pop("PYTHONPATH", None)
    probe = subprocess.run(
        [sys.executable, "-c", "import paged_kv_cache_resolve_amd as pk\n"
         "try:\n    pk.library()\nexcept ImportError as e:\n    print('missing:', e)\n"],
        cwd=tmp_path, env=env, capture_output=True, text=True, timeout=300)
    assert probe.returncode == 0, probe.stderr
    assert "missing:" in probe.stdout and "paged_kv_cache_resolve_amd.build" in probe.stdout
    r = subprocess.run([sys.executable, "-m", "paged_kv_cache_resolve_amd.build"], cwd=tmp_path,
                       env=env, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, r.stderr[-2000:]
    assert (tmp_path / "paged_kv_cache_resolve_amd" / "libpagedkv.so").exists()


def test_binding_refuses_host_tensors():
    import torch
    with pytest.raises(ValueError):
        pk.kv_pool_create(4, 16, 1, 2, 64, torch.bfloat16, device="cpu")
    data = torch.zeros((4, 2, 1, 2, 16, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        pk.KVPool(4, 16, 1, 2, 64, torch.bfloat16, data=data)


def test_validate_decode_inputs_host_helper():
    import torch
    t = torch.tensor([[3, 1, -7], [0, 2, 99]], dtype=torch.int32)
    pk.validate_decode_inputs(4, 4, t, torch.tensor([8, 6], dtype=torch.int32))
    pk.validate_decode_inputs(4, 4, t, torch.tensor([8, 6], dtype=torch.int32),
                              positions=torch.tensor([7, -1], dtype=torch.int32))
    bad = [
        (t, [13, 6], None),                                               # past the table
        (torch.tensor([[3, 4, 0], [0, 2, 0]], dtype=torch.int32), [8, 6], None),   # block 4 of 4
        (torch.tensor([[3, 1, 0], [1, 2, 0]], dtype=torch.int32), [8, 6], None),   # shared block
        (t, [-1, 6], None),
        (t, [8, 6], [12, -1]),                                            # block of 12 is -7
        (t, [8, 6], [7, 12]),                                             # 12 // 4 = 3: past the row
    ]
    for tab, lens, pos in bad:
        with pytest.raises(ValueError):
            pk.validate_decode_inputs(4, 4, tab, torch.tensor(lens, dtype=torch.int32),
                                      None if pos is None else torch.tensor(pos, dtype=torch.int32))
