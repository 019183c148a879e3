"""Paged-KV-cache attention decode on AMD Instinct MI355X (gfx950).

Thin Python binding over libpagedkv.so: it checks tensors (device, dtype,
shape, contiguity), passes their device pointers and the current HIP stream
to the C ABI, and raises on a non-zero status.  Every step of the path runs
in the library's HIP kernels; PyTorch only supplies device memory and
streams.

    pool = kv_pool_create(num_blocks, block_size, layers, kv_heads, head_dim, dtype)
    kv_append(pool, layer, k_new, v_new, block_tables, positions)
    paged_attention_decode(out, q, pool, layer, block_tables, context_lens, scale)
    paged_attention_decode_append(out, q, pool, layer, block_tables, context_lens, scale,
                                  k_new, v_new, positions)   # both of the above in one call
    k_all, v_all, mask = paged_kv_gather(pool, layer, block_tables, context_lens, max_len)

    mgr = BlockManager(pool, max_blocks_per_seq)   # host block manager (C++)
    mgr.add_sequence(7); starts = mgr.reserve([7], [prompt_len])
    tables, lens = mgr.block_tables([7])            # host int32 arrays
"""

from __future__ import annotations

import ctypes
import threading

import numpy as np
import torch

from . import _lib
from ._lib import OutOfBlocksError, PagedKVError  # noqa: F401

# The library is loaded on first use (so that the build module imports on a
# tree where it has not been built yet); a missing library raises there.
_L = _lib.LazyLib()

__all__ = [
    "KVPool", "kv_pool_create", "BlockManager", "kv_append", "kv_append_layers", "kv_append_tokens",
    "paged_kv_gather", "paged_attention_decode",
    "paged_attention_decode_append", "DecodePlan", "dense_attention_decode",
    "paged_attention_workspace_bytes", "paged_kv_resolve", "validate_decode_inputs",
    "split_mode", "SPLIT_AUTO", "SPLIT_CHUNKS",
    "PagedKVError", "OutOfBlocksError",
    "library",
]

# decode work split, passed to the library as per-call flags
SPLIT_AUTO = 0                      # per-pair workgroups for small batches, else the chunk split
SPLIT_CHUNKS = _lib.DECODE_CHUNKS   # always the persistent chunk split

_DTYPES = {torch.float32: _lib.F32, torch.bfloat16: _lib.BF16, torch.float16: _lib.F16}


def library() -> ctypes.CDLL:
    """The loaded libpagedkv.so (loads it if needed)."""
    return _lib.lib()


def _check(status: int, what: str) -> None:
    if status == _lib.OK:
        return
    if status == _lib.ERR_OUT_OF_BLOCKS:
        raise OutOfBlocksError(status, what)
    raise PagedKVError(status, what)


_split_default = threading.local()


def _split_flags(split) -> int:
    """Decode flags for `split` (SPLIT_AUTO, SPLIT_CHUNKS, "auto", "chunks";
    None = this thread's default, set by the split_mode context manager)."""
    if split is None:
        return getattr(_split_default, "flags", SPLIT_AUTO)
    if split in ("auto", SPLIT_AUTO):
        return SPLIT_AUTO
    if split in ("chunks", SPLIT_CHUNKS):
        return SPLIT_CHUNKS
    raise ValueError(f"unknown split {split!r}")


# The checks below run on every call, so they use the cheapest tensor
# queries (device index as an int, torch.Size compared as a tuple) and hand
# ctypes plain integers for pointers.

def _stream(device: torch.device) -> int:
    """The current HIP stream of `device`, as an integer handle."""
    return torch.cuda.current_stream(device).cuda_stream


def _dev_tensor(t: torch.Tensor, name: str, device: torch.device, dtype=None, shape=None) -> int:
    """Check a tensor argument and return its device address."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda or t.get_device() != device.index:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and t.shape != shape:
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


class KVPool:
    """One preallocated pool of fixed-size KV blocks in device memory
    ([num_blocks, 2 (K/V), layers, kv_heads, block_size, head_dim]) plus the
    library's host free-block stack."""

    def __init__(self, num_blocks: int, block_size: int = 16, layers: int = 24,
                 kv_heads: int = 2, head_dim: int = 64, dtype: torch.dtype = torch.bfloat16,
                 device="cuda", data: torch.Tensor | None = None):
        if dtype not in _DTYPES:
            raise ValueError(f"unsupported dtype {dtype}")
        self.num_blocks, self.block_size, self.layers = num_blocks, block_size, layers
        self.kv_heads, self.head_dim, self.dtype = kv_heads, head_dim, dtype
        shape = (num_blocks, 2, layers, kv_heads, block_size, head_dim)
        if data is None:
            device = torch.device(device)
            if device.type != "cuda":
                raise ValueError("the pool must live in GPU memory")
            data = torch.zeros(shape, dtype=dtype, device=device)
        if data.device.type != "cuda":
            raise ValueError("the pool must live in GPU memory")
        self.device = torch.device("cuda", data.get_device())
        _dev_tensor(data, "data", self.device, dtype, shape)
        self.data = data
        self._handle = ctypes.c_void_p()
        nbytes = data.numel() * data.element_size()
        _check(_L.kv_pool_create(ctypes.byref(self._handle), num_blocks, block_size, layers,
                                 kv_heads, head_dim, _DTYPES[dtype], ctypes.c_void_p(data.data_ptr()),
                                 nbytes), "kv_pool_create")

    @property
    def handle(self) -> ctypes.c_void_p:
        return self._handle

    def allocate_block(self) -> int:
        out = ctypes.c_int32()
        _check(_L.kv_pool_alloc_block(self._handle, ctypes.byref(out)), "kv_pool_alloc_block")
        return out.value

    def free_block(self, block_id: int) -> None:
        _check(_L.kv_pool_free_block(self._handle, int(block_id)), "kv_pool_free_block")

    @property
    def num_free(self) -> int:
        n = _L.kv_pool_num_free(self._handle)
        _check(min(n, 0), "kv_pool_num_free")
        return n

    def __del__(self):
        h = getattr(self, "_handle", None)
        # at interpreter exit the module globals may already be cleared
        if h is not None and h.value and _L is not None:
            _L.kv_pool_destroy(h)
            self._handle = ctypes.c_void_p()


class BlockManager:
    """Host block manager over a pool's free-block stack (libpagedkv's C++
    manager): admission of a step, tail-block allocation as sequences grow,
    release of a finished sequence's blocks, and waste statistics.  Host
    memory only.  Sequence ids are caller-chosen integers."""

    def __init__(self, pool: KVPool, max_blocks_per_seq: int):
        self.pool = pool                      # keeps the pool alive
        self.max_blocks_per_seq = int(max_blocks_per_seq)
        self._handle = ctypes.c_void_p()
        _check(_L.kv_manager_create(ctypes.byref(self._handle), pool.handle,
                                    self.max_blocks_per_seq), "kv_manager_create")

    @staticmethod
    def _ids(seq_ids):
        return np.ascontiguousarray(np.asarray(seq_ids, dtype=np.int64).reshape(-1))

    def add_sequence(self, seq_id: int) -> None:
        _check(_L.kv_manager_add_sequence(self._handle, int(seq_id)), "kv_manager_add_sequence")

    def blocks_needed(self, seq_ids, counts) -> int:
        ids = self._ids(seq_ids)
        cnt = np.ascontiguousarray(np.asarray(counts, dtype=np.int32).reshape(-1))
        if cnt.shape != ids.shape:
            raise ValueError("seq_ids and counts differ in length")
        n = _L.kv_manager_blocks_needed(self._handle, len(ids), ids.ctypes.data, cnt.ctypes.data)
        _check(int(min(n, 0)), "kv_manager_blocks_needed")
        return int(n)

    def reserve(self, seq_ids, counts) -> np.ndarray:
        """Admit a step (grow seq_ids[i] by counts[i] tokens) and return each
        sequence's first new position; OutOfBlocksError leaves all unchanged."""
        ids = self._ids(seq_ids)
        cnt = np.ascontiguousarray(np.asarray(counts, dtype=np.int32).reshape(-1))
        if cnt.shape != ids.shape:
            raise ValueError("seq_ids and counts differ in length")
        starts = np.empty(len(ids), dtype=np.int32)
        _check(_L.kv_manager_reserve(self._handle, len(ids), ids.ctypes.data, cnt.ctypes.data,
                                     starts.ctypes.data), "kv_manager_reserve")
        return starts

    def release(self, seq_id: int) -> None:
        _check(_L.kv_manager_release(self._handle, int(seq_id)), "kv_manager_release")

    def block_tables(self, seq_ids) -> tuple[np.ndarray, np.ndarray]:
        """Host int32 [n, max_blocks_per_seq] tables (-1 padded) and [n] lengths."""
        ids = self._ids(seq_ids)
        tables = np.empty((len(ids), self.max_blocks_per_seq), dtype=np.int32)
        lens = np.empty(len(ids), dtype=np.int32)
        _check(_L.kv_manager_block_tables(self._handle, len(ids), ids.ctypes.data,
                                          tables.ctypes.data, lens.ctypes.data),
               "kv_manager_block_tables")
        return tables, lens

    def stats(self) -> dict:
        st = _lib.ManagerStats()
        _check(_L.kv_manager_stats(self._handle, ctypes.byref(st)), "kv_manager_stats")
        return {name: getattr(st, name) for name, _ in st._fields_}

    def close(self) -> None:
        """Return every live sequence's blocks to the pool and free the
        manager (also done when the object is collected)."""
        h = getattr(self, "_handle", None)
        # at interpreter exit the module globals may already be cleared
        if h is not None and h.value and _L is not None:
            _L.kv_manager_destroy(h)
            self._handle = ctypes.c_void_p()

    def __del__(self):
        self.close()


def validate_decode_inputs(num_blocks: int, block_size: int, block_tables: torch.Tensor,
                           context_lens: torch.Tensor, positions: torch.Tensor | None = None) -> None:
    """Check the device-resident inputs the library trusts (it cannot read
    them without a synchronisation): 0 <= T_b <= max_blocks_per_seq *
    block_size, every used table entry a block of the pool, no physical
    block used twice, and for an append every non-negative position inside
    the table with its block present.  Copies the arrays to the host (a
    synchronisation); meant for tests and debugging.  Raises ValueError."""
    tables = block_tables.detach().cpu().numpy()
    lens = context_lens.detach().cpu().numpy().astype(np.int64)
    if tables.ndim != 2 or lens.shape != (tables.shape[0],):
        raise ValueError("block_tables must be [batch, max_blocks_per_seq], context_lens [batch]")
    mb = tables.shape[1]
    if (lens < 0).any() or (lens > mb * block_size).any():
        raise ValueError("a context length lies outside [0, max_blocks_per_seq * block_size]")
    used = (lens + block_size - 1) // block_size
    cols = np.arange(mb)[None, :] < used[:, None]
    ids = tables[cols]
    if ((ids < 0) | (ids >= num_blocks)).any():
        raise ValueError("a used block-table entry lies outside the pool")
    if len(np.unique(ids)) != len(ids):
        raise ValueError("a physical block is used by two logical blocks")
    if positions is not None:
        pos = positions.detach().cpu().numpy().astype(np.int64)
        if pos.shape != lens.shape:
            raise ValueError("positions must be [batch]")
        live = pos >= 0
        if (pos[live] >= mb * block_size).any():
            raise ValueError("a position lies past the block table")
        blk = tables[np.nonzero(live)[0], pos[live] // block_size]
        if ((blk < 0) | (blk >= num_blocks)).any():
            raise ValueError("the block of an appended position is missing")


def kv_pool_create(num_blocks: int, block_size: int = 16, layers: int = 24, kv_heads: int = 2,
                   head_dim: int = 64, dtype: torch.dtype = torch.bfloat16,
                   device="cuda") -> KVPool:
    """Preallocate a zero-filled pool on the GPU and describe it to the library."""
    return KVPool(num_blocks, block_size, layers, kv_heads, head_dim, dtype, device)


def _tables_args(pool, block_tables, batch):
    if block_tables.dim() != 2 or block_tables.shape[0] != batch:
        raise ValueError("block_tables must be [batch, max_blocks_per_seq]")
    return _dev_tensor(block_tables, "block_tables", pool.device, torch.int32), int(block_tables.shape[1])


def kv_append(pool: KVPool, layer: int, k_new: torch.Tensor, v_new: torch.Tensor,
              block_tables: torch.Tensor, positions: torch.Tensor) -> None:
    """Write k_new/v_new [batch, kv_heads, head_dim] at token positions[b]."""
    batch = int(positions.shape[0])
    shape = (batch, pool.kv_heads, pool.head_dim)
    kp = _dev_tensor(k_new, "k_new", pool.device, pool.dtype, shape)
    vp = _dev_tensor(v_new, "v_new", pool.device, pool.dtype, shape)
    tp, mb = _tables_args(pool, block_tables, batch)
    pp = _dev_tensor(positions, "positions", pool.device, torch.int32, (batch,))
    _check(_L.kv_append(pool.handle, layer, kp, vp, tp, mb, pp, batch, _stream(pool.device)),
           "kv_append")


def kv_append_layers(pool: KVPool, k_new: torch.Tensor, v_new: torch.Tensor,
                     block_tables: torch.Tensor, positions: torch.Tensor) -> None:
    """Write k_new/v_new [batch, layers, kv_heads, head_dim] at token
    positions[b] for every layer in one launch."""
    batch = int(positions.shape[0])
    shape = (batch, pool.layers, pool.kv_heads, pool.head_dim)
    kp = _dev_tensor(k_new, "k_new", pool.device, pool.dtype, shape)
    vp = _dev_tensor(v_new, "v_new", pool.device, pool.dtype, shape)
    tp, mb = _tables_args(pool, block_tables, batch)
    pp = _dev_tensor(positions, "positions", pool.device, torch.int32, (batch,))
    _check(_L.kv_append_layers(pool.handle, kp, vp, tp, mb, pp, batch, _stream(pool.device)),
           "kv_append_layers")


def kv_append_tokens(pool: KVPool, layer: int, k_new: torch.Tensor, v_new: torch.Tensor,
                     block_tables: torch.Tensor, start_positions: torch.Tensor,
                     token_offsets: torch.Tensor) -> None:
    """Write several tokens per sequence: rows token_offsets[b] ..
    token_offsets[b+1]-1 of k_new/v_new [total, kv_heads, head_dim] go to
    positions start_positions[b], start_positions[b] + 1, ..."""
    batch = int(start_positions.shape[0])
    total = int(k_new.shape[0]) if k_new.dim() == 3 else -1
    shape = (total, pool.kv_heads, pool.head_dim)
    kp = _dev_tensor(k_new, "k_new", pool.device, pool.dtype, shape)
    vp = _dev_tensor(v_new, "v_new", pool.device, pool.dtype, shape)
    tp, mb = _tables_args(pool, block_tables, batch)
    sp = _dev_tensor(start_positions, "start_positions", pool.device, torch.int32, (batch,))
    op = _dev_tensor(token_offsets, "token_offsets", pool.device, torch.int32, (batch + 1,))
    _check(_L.kv_append_tokens(pool.handle, layer, kp, vp, tp, mb, sp, op, batch, total,
                               _stream(pool.device)), "kv_append_tokens")


def paged_kv_gather(pool: KVPool, layer: int, block_tables: torch.Tensor,
                    context_lens: torch.Tensor, max_len: int | None = None, out=None):
    """Gather every sequence's K/V into contiguous [batch, max_len, kv_heads,
    head_dim] tensors plus a uint8 [batch, max_len] mask (1 = cached token).
    ``max_len`` defaults to max(context_lens) (read back from the device)."""
    batch = int(context_lens.shape[0])
    if max_len is None:
        max_len = int(context_lens.max().item()) if batch else 0
    shape = (batch, max_len, pool.kv_heads, pool.head_dim)
    if out is None:
        k = torch.empty(shape, dtype=pool.dtype, device=pool.device)
        v = torch.empty(shape, dtype=pool.dtype, device=pool.device)
        mask = torch.empty((batch, max_len), dtype=torch.uint8, device=pool.device)
    else:
        k, v, mask = out
    kp = _dev_tensor(k, "k_out", pool.device, pool.dtype, shape)
    vp = _dev_tensor(v, "v_out", pool.device, pool.dtype, shape)
    mp = _dev_tensor(mask, "mask", pool.device, torch.uint8, (batch, max_len))
    tp, mb = _tables_args(pool, block_tables, batch)
    lp = _dev_tensor(context_lens, "context_lens", pool.device, torch.int32, (batch,))
    _check(_L.paged_kv_gather(kp, vp, mp, pool.handle, layer, tp, mb, lp, batch, max_len,
                              _stream(pool.device)), "paged_kv_gather")
    return k, v, mask


def paged_attention_workspace_bytes(pool: KVPool, batch: int, num_q_heads: int) -> int:
    """Device workspace bytes of a decode of this shape (the library's own
    query: the size depends on the pool's dtype, block size and head shape)."""
    n = _L.paged_attention_workspace_bytes(pool.handle, batch, num_q_heads)
    if n == 0 and batch >= 0:
        raise PagedKVError(_lib.ERR_INVALID_ARG, "paged_attention_workspace_bytes")
    return n


_WORKSPACES: dict = {}


def _workspace(device: torch.device, nbytes: int, stream: int) -> torch.Tensor:
    key = (device.index, stream)
    ws = _WORKSPACES.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(nbytes, 1 << 20), dtype=torch.uint8, device=device)
        _WORKSPACES[key] = ws
    return ws


def _decode_args(out, q, pool, block_tables, context_lens, workspace):
    if q.dim() != 3:
        raise ValueError("q must be [batch, num_q_heads, head_dim]")
    batch, hq, d = (int(x) for x in q.shape)
    if d != pool.head_dim:
        raise ValueError("q head_dim does not match the pool")
    qp = _dev_tensor(q, "q", pool.device, pool.dtype)
    op = _dev_tensor(out, "out", pool.device, pool.dtype, q.shape)
    tp, mb = _tables_args(pool, block_tables, batch)
    lp = _dev_tensor(context_lens, "context_lens", pool.device, torch.int32, (batch,))
    need = paged_attention_workspace_bytes(pool, batch, hq)
    stream = _stream(pool.device)
    if workspace is None:
        workspace = _workspace(pool.device, need, stream)
    wp = _dev_tensor(workspace, "workspace", pool.device, torch.uint8)
    return batch, hq, qp, op, tp, mb, lp, wp, workspace.numel(), stream


def paged_attention_decode(out: torch.Tensor, q: torch.Tensor, pool: KVPool, layer: int,
                           block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float,
                           workspace: torch.Tensor | None = None, split=None) -> torch.Tensor:
    """out[b, h] = softmax_t(scale * q[b, h] . K_t) V_t over the T_b cached
    tokens of sequence b, resolved through its block table.  q and out are
    [batch, num_q_heads, head_dim] in the pool dtype.  A workspace is taken
    from a per-stream cache unless one is given.  `split`: SPLIT_AUTO or
    SPLIT_CHUNKS (None = the thread's default, see split_mode)."""
    batch, hq, qp, op, tp, mb, lp, wp, wn, stream = _decode_args(out, q, pool, block_tables,
                                                                 context_lens, workspace)
    _check(_L.paged_attention_decode(op, qp, pool.handle, layer, tp, mb, lp, batch, hq, scale,
                                     wp, wn, _split_flags(split), stream),
           "paged_attention_decode")
    return out


def paged_attention_decode_append(out: torch.Tensor, q: torch.Tensor, pool: KVPool, layer: int,
                                  block_tables: torch.Tensor, context_lens: torch.Tensor,
                                  scale: float, k_new: torch.Tensor, v_new: torch.Tensor,
                                  positions: torch.Tensor,
                                  workspace: torch.Tensor | None = None,
                                  split=None) -> torch.Tensor:
    """kv_append(pool, layer, k_new, v_new, block_tables, positions) followed
    by paged_attention_decode(out, q, ...), as one library call (the decode
    kernel reads the new rows from k_new / v_new where it can, saving the
    separate append launch)."""
    batch, hq, qp, op, tp, mb, lp, wp, wn, stream = _decode_args(out, q, pool, block_tables,
                                                                 context_lens, workspace)
    shape = (batch, pool.kv_heads, pool.head_dim)
    kp = _dev_tensor(k_new, "k_new", pool.device, pool.dtype, shape)
    vp = _dev_tensor(v_new, "v_new", pool.device, pool.dtype, shape)
    pp = _dev_tensor(positions, "positions", pool.device, torch.int32, (batch,))
    _check(_L.paged_attention_decode_append(op, qp, kp, vp, pp, pool.handle, layer, tp, mb, lp,
                                            batch, hq, scale, wp, wn, _split_flags(split),
                                            stream),
           "paged_attention_decode_append")
    return out


class DecodePlan:
    """A decode step whose tensors are fixed: they are checked once here, and
    run() only passes their addresses and the current stream to the library.
    For loops that reuse the same buffers every step (update their contents
    in place).  With k_new, v_new and positions the step is
    paged_attention_decode_append, otherwise paged_attention_decode.  The
    plan holds references to the tensors, so their storage stays alive."""

    def __init__(self, out: torch.Tensor, q: torch.Tensor, pool: KVPool, layer: int,
                 block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float,
                 k_new: torch.Tensor | None = None, v_new: torch.Tensor | None = None,
                 positions: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                 split=None):
        append = k_new is not None or v_new is not None or positions is not None
        if append and (k_new is None or v_new is None or positions is None):
            raise ValueError("k_new, v_new and positions go together")
        batch, hq, qp, op, tp, mb, lp, wp, wn, stream = _decode_args(out, q, pool, block_tables,
                                                                     context_lens, workspace)
        self.pool = pool
        self._keep = (out, q, block_tables, context_lens, k_new, v_new, positions,
                      workspace if workspace is not None else _workspace(pool.device, wn, stream))
        self._device = pool.device
        # the shared per-stream workspace may only be used on its own stream
        self._stream = None if workspace is not None else stream
        if append:
            shape = (batch, pool.kv_heads, pool.head_dim)
            kp = _dev_tensor(k_new, "k_new", pool.device, pool.dtype, shape)
            vp = _dev_tensor(v_new, "v_new", pool.device, pool.dtype, shape)
            pp = _dev_tensor(positions, "positions", pool.device, torch.int32, (batch,))
            self._fn = _L.paged_attention_decode_append
            self._args = (op, qp, kp, vp, pp, pool.handle, layer, tp, mb, lp, batch, hq,
                          float(scale), wp, wn, _split_flags(split))
            self._what = "paged_attention_decode_append"
        else:
            self._fn = _L.paged_attention_decode
            self._args = (op, qp, pool.handle, layer, tp, mb, lp, batch, hq, float(scale), wp, wn,
                          _split_flags(split))
            self._what = "paged_attention_decode"

    def run(self) -> torch.Tensor:
        """Enqueue the step on the current stream; returns `out`.  Without an
        explicit workspace the plan uses the stream's cached one, so it must
        run on the stream that was current when it was built."""
        stream = torch.cuda.current_stream(self._device).cuda_stream
        if self._stream is not None and stream != self._stream:
            raise RuntimeError("DecodePlan built on another stream; pass a workspace to share it")
        _check(self._fn(*self._args, stream), self._what)
        return self._keep[0]


def dense_attention_decode(out: torch.Tensor, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                           mask: torch.Tensor, scale: float, workspace=None) -> torch.Tensor:
    """Decode over gathered, padded K/V (what paged_kv_gather returns): k and
    v [batch, max_len, kv_heads, head_dim], mask uint8 [batch, max_len]
    (token t of sequence b attended iff mask[b, t] != 0).  Every max_len row
    is read.  bf16 and fp16."""
    if q.dim() != 3 or k.dim() != 4:
        raise ValueError("q must be [batch, num_q_heads, head_dim], k [batch, max_len, kv_heads, head_dim]")
    if q.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {q.dtype}")
    if not q.is_cuda:
        raise ValueError("q must be a GPU tensor")
    device = torch.device("cuda", q.get_device())
    batch, hq, d = (int(x) for x in q.shape)
    _, max_len, hkv, _ = (int(x) for x in k.shape)
    shape = (batch, max_len, hkv, d)
    qp = _dev_tensor(q, "q", device, q.dtype)
    op = _dev_tensor(out, "out", device, q.dtype, q.shape)
    kp = _dev_tensor(k, "k", device, q.dtype, shape)
    vp = _dev_tensor(v, "v", device, q.dtype, shape)
    mp = _dev_tensor(mask, "mask", device, torch.uint8, (batch, max_len))
    need = _L.dense_attention_workspace_bytes(batch, hkv, hq, d)
    if need == 0:
        raise ValueError("num_q_heads must be a multiple of kv_heads")
    stream = _stream(device)
    if workspace is None:
        workspace = _workspace(device, need, stream)
    wp = _dev_tensor(workspace, "workspace", device, torch.uint8)
    _check(_L.dense_attention_decode(op, qp, kp, vp, mp, batch, max_len, hkv, d, hq,
                                     _DTYPES[q.dtype], ctypes.c_float(scale), wp,
                                     workspace.numel(), stream), "dense_attention_decode")
    return out


def paged_kv_resolve(block_tables: torch.Tensor, context_lens: torch.Tensor, block_size: int,
                     max_len: int) -> torch.Tensor:
    """int64 [batch, max_len] global slot ids (physical block * block_size +
    offset), -1 past each sequence's length."""
    device = block_tables.device
    batch = int(context_lens.shape[0])
    slots = torch.empty((batch, max_len), dtype=torch.int64, device=device)
    sp = _dev_tensor(slots, "slots", device, torch.int64)
    if block_tables.dim() != 2 or block_tables.shape[0] != batch:
        raise ValueError("block_tables must be [batch, max_blocks_per_seq]")
    tp = _dev_tensor(block_tables, "block_tables", device, torch.int32)
    lp = _dev_tensor(context_lens, "context_lens", device, torch.int32, (batch,))
    _check(_L.paged_kv_resolve(sp, tp, int(block_tables.shape[1]), lp, batch, block_size, max_len,
                               _stream(device)), "paged_kv_resolve")
    return slots


class split_mode:
    """Context manager: decode calls made by this thread inside it that pass
    no `split` use `mode` (SPLIT_AUTO or SPLIT_CHUNKS).  The setting is
    per thread and lives in the binding only: the library takes the split as
    a per-call flag, so other threads' calls are not affected."""

    def __init__(self, mode):
        self.flags = _split_flags(mode)
        self.prev = None

    def __enter__(self):
        self.prev = getattr(_split_default, "flags", SPLIT_AUTO)
        _split_default.flags = self.flags
        return self

    def __exit__(self, *exc):
        _split_default.flags = self.prev
        return False
