"""Plain float64 reference for the paged-KV decode path (test infrastructure).

Sources (three web pages on paged KV caches):
  [vllmini]   "vllmini: Building a Minimalist PagedAttention and KV Cache
              Engine" -- sections "PagedAttention Metaphor", "The CUDA Block
              Kernel".
  [kv-cache]  "KV Cache and Attention Mechanisms: PagedAttention and vLLM" --
              section 2 "PagedAttention Architecture".
  [mini-infer] "Paged KV-Cache Memory Management" -- sections "The Problem",
              "The Solution", "Memory Waste Analysis", "Python
              Implementation: Physical Block Pool & Batched Paging",
              "Zero-Copy Batched Attention Gather".

Storage conventions: a pool is a numpy array of shape
``[num_blocks, 2, layers, kv_heads, block_size, head_dim]`` (K at index 0 of
the second axis, V at index 1), holding float32 values or bfloat16 bit
patterns as uint16 (fp16 as numpy float16).  Copies (gather, append) move raw storage; attention
widens to float64 first.

Readings taken where the pages leave a step open:
  * Attention is softmax(scale * q K^T) V over all T_b cached tokens of the
    sequence (decode: the query is the newest token, so no causal mask).
  * Query head h reads KV head h // (Hq / Hkv) (contiguous head groups).
  * context_lens counts the token appended in the same step.
  * T_b = 0 yields a zero output row.
  * A block table row is shared by all heads and layers of its sequence;
    entries past ceil(T_b / block_size) are never read.
"""

from __future__ import annotations

import math

import numpy as np


# ----------------------------------------------------------------------------
# Storage helpers
# ----------------------------------------------------------------------------

def widen(x: np.ndarray, dtype: str) -> np.ndarray:
    """Raw storage -> float64.  bfloat16 is the upper half of a float32, so
    widening is exact: shift the 16 stored bits into the high half.  IEEE
    half precision (numpy float16) widens exactly by conversion."""
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        hi = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return hi.view(np.float32).astype(np.float64)
    if dtype == "f16":
        return np.asarray(x, dtype=np.float16).astype(np.float64)
    raise ValueError(dtype)


# ----------------------------------------------------------------------------
# Block-table resolution
# ----------------------------------------------------------------------------

def logical_to_physical(table_row: np.ndarray, t: int, block_size: int) -> tuple[int, int]:
    """Token t of a sequence lives in logical block t // block_size at offset
    t % block_size; the sequence's block table maps that logical block to a
    physical block id.

    [vllmini] "PagedAttention Metaphor" (logical blocks mapped to
    non-contiguous physical pages through a page table, resolved on the fly);
    [mini-infer] "The Solution" (block table: logical block -> physical id,
    B tokens per block).
    """
    return int(table_row[t // block_size]), t % block_size


def resolve_slots(block_tables: np.ndarray, context_lens: np.ndarray,
                  block_size: int, max_len: int) -> np.ndarray:
    """int64 [S, max_len]: global slot index phys * block_size + offset for
    every cached token, -1 for positions at or past the sequence's length.

    Same sources as :func:`logical_to_physical`.
    """
    S = len(context_lens)
    out = np.full((S, max_len), -1, dtype=np.int64)
    for b in range(S):
        T = int(context_lens[b])
        if T > max_len:
            raise ValueError("max_len shorter than a sequence")
        for t in range(T):
            phys, off = logical_to_physical(block_tables[b], t, block_size)
            out[b, t] = phys * block_size + off
    return out


# ----------------------------------------------------------------------------
# Gather
# ----------------------------------------------------------------------------

def gather_sequence(pool: np.ndarray, layer: int, table_row: np.ndarray, T: int
                    ) -> tuple[np.ndarray, np.ndarray]:
    """Contiguous raw K and V, each [T, kv_heads, head_dim], of one sequence
    at one layer.

    [mini-infer] "Python Implementation: Physical Block Pool" (pool layout
    [num_blocks, 2 (K/V), num_layers, num_kv_heads, block_size, head_dim])
    and "Zero-Copy Batched Attention Gather" (past K/V of a sequence gathered
    from its physical blocks).
    """
    block_size = pool.shape[4]
    if T == 0:
        empty = pool[:0, 0, 0, :, 0, :]          # shape [0, Hkv, D]
        return empty.copy(), empty.copy()
    phys_off = [logical_to_physical(table_row, t, block_size) for t in range(T)]
    phys = np.array([p for p, _ in phys_off], dtype=np.int64)
    off = np.array([o for _, o in phys_off], dtype=np.int64)
    K = np.stack([pool[phys[t], 0, layer, :, off[t], :] for t in range(T)])
    V = np.stack([pool[phys[t], 1, layer, :, off[t], :] for t in range(T)])
    return K, V


def paged_kv_gather(pool: np.ndarray, layer: int, block_tables: np.ndarray,
                    context_lens: np.ndarray, max_len: int
                    ) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Batched gather into contiguous ``k_out, v_out [S, max_len, Hkv, D]``
    plus ``mask uint8 [S, max_len]`` (1 = cached token, 0 = padding).
    Padding positions hold zero bits.

    [mini-infer] "Zero-Copy Batched Attention Gather": past keys and values of
    all active decode sequences gathered from the physical blocks into one
    contiguous batch tensor with a mask.
    """
    S = len(context_lens)
    Hkv, D = pool.shape[3], pool.shape[5]
    k_out = np.zeros((S, max_len, Hkv, D), dtype=pool.dtype)
    v_out = np.zeros((S, max_len, Hkv, D), dtype=pool.dtype)
    mask = np.zeros((S, max_len), dtype=np.uint8)
    for b in range(S):
        T = int(context_lens[b])
        if T > max_len:
            raise ValueError("max_len shorter than a sequence")
        K, V = gather_sequence(pool, layer, block_tables[b], T)
        k_out[b, :T] = K
        v_out[b, :T] = V
        mask[b, :T] = 1
    return k_out, v_out, mask


# ----------------------------------------------------------------------------
# Append
# ----------------------------------------------------------------------------

def kv_append(pool: np.ndarray, layer: int, block_tables: np.ndarray,
              positions: np.ndarray, k_new: np.ndarray, v_new: np.ndarray,
              *, in_place: bool = False) -> np.ndarray:
    """Write each sequence's new token K/V ([S, Hkv, D]) into the slot of
    token ``positions[b]``: the tail block of the sequence.  A negative
    position leaves that sequence untouched.

    [kv-cache] section 2 "PagedAttention Architecture" (blocks allocated per
    block as generation proceeds; only the final block is partly filled);
    [mini-infer] "The Solution" (each physical block stores B tokens of K and
    V for all layers).
    """
    out = pool if in_place else pool.copy()
    block_size = pool.shape[4]
    for b in range(len(positions)):
        pos = int(positions[b])
        if pos < 0:
            continue
        phys, off = logical_to_physical(block_tables[b], pos, block_size)
        out[phys, 0, layer, :, off, :] = k_new[b]
        out[phys, 1, layer, :, off, :] = v_new[b]
    return out


def kv_append_layers(pool: np.ndarray, block_tables: np.ndarray, positions: np.ndarray,
                     k_new: np.ndarray, v_new: np.ndarray, *, in_place: bool = False
                     ) -> np.ndarray:
    """One token per sequence for every layer at once: k_new and v_new are
    [S, L, Hkv, D]; layer l of sequence b goes where kv_append(layer=l)
    would put it.  A negative position leaves that sequence untouched.

    [mini-infer] "The Solution" (a physical block holds B tokens of K and V
    for all layers, so one slot serves every layer of a token).
    """
    out = pool if in_place else pool.copy()
    for layer in range(pool.shape[2]):
        kv_append(out, layer, block_tables, positions, k_new[:, layer], v_new[:, layer],
                  in_place=True)
    return out


def kv_append_tokens(pool: np.ndarray, layer: int, block_tables: np.ndarray,
                     start_positions: np.ndarray, token_offsets: np.ndarray,
                     k_new: np.ndarray, v_new: np.ndarray, *, in_place: bool = False
                     ) -> np.ndarray:
    """Several consecutive tokens per sequence (a prompt, or a chunk of one):
    rows token_offsets[b] .. token_offsets[b+1]-1 of k_new / v_new ([N, Hkv,
    D]) are the tokens of sequence b, and row token_offsets[b] + i goes to
    logical position start_positions[b] + i, resolved through the block
    table.  A negative start position leaves that sequence untouched.

    [kv-cache] section 2 (a prompt fills whole blocks, only the last one is
    partly filled); [vllmini] "PagedAttention Metaphor" (logical positions
    resolve to physical slots through the table).
    """
    out = pool if in_place else pool.copy()
    block_size = pool.shape[4]
    for b in range(len(start_positions)):
        start = int(start_positions[b])
        if start < 0:
            continue
        for row in range(int(token_offsets[b]), int(token_offsets[b + 1])):
            t = start + row - int(token_offsets[b])
            phys, off = logical_to_physical(block_tables[b], t, block_size)
            out[phys, 0, layer, :, off, :] = k_new[row]
            out[phys, 1, layer, :, off, :] = v_new[row]
    return out


# ----------------------------------------------------------------------------
# Attention
# ----------------------------------------------------------------------------

def kv_head_of(h: int, num_q_heads: int, num_kv_heads: int) -> int:
    """Grouped-query mapping: consecutive groups of Hq / Hkv query heads
    share one KV head (the pages show one head count only; this is the
    plainest reading that covers Hq != Hkv)."""
    return h // (num_q_heads // num_kv_heads)


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """One decode step for one sequence, float64.

    q [Hq, D]; K, V [T, Hkv, D].  For each query head: scores
    s_t = scale * <q_h, K_t>, weights exp(s_t - max s) normalised to sum 1,
    output = weighted sum of the V rows.  T = 0 gives zeros.

    [vllmini] "The CUDA Block Kernel" (dot-product attention scores computed
    over the resolved pages) and the page's introduction (each generation step
    reads the K/V of all past tokens to compute attention weights).
    """
    Hq, D = q.shape
    T, Hkv, _ = K.shape
    out = np.zeros((Hq, D), dtype=np.float64)
    if T == 0:
        return out
    for h in range(Hq):
        g = kv_head_of(h, Hq, Hkv)
        s = scale * (K[:, g, :] @ q[h])
        w = np.exp(s - s.max())
        out[h] = (w / w.sum()) @ V[:, g, :]
    return out


def validate_decode_inputs(num_blocks: int, block_size: int, block_tables: np.ndarray,
                           context_lens: np.ndarray, num_q_heads: int, num_kv_heads: int) -> None:
    """The preconditions of a decode: query heads a multiple of KV heads,
    0 <= T_b <= max_blocks_per_seq * B, every used table entry a block of the
    pool, and no physical block used by two (sequence, logical block) pairs
    (so no two tokens share a slot).  Raises ValueError.

    [vllmini] "PagedAttention Metaphor" (each logical block maps to its own
    physical block); [mini-infer] "The Solution" (the table maps a request's
    logical blocks to physical block ids of the pool).
    """
    if num_kv_heads < 1 or num_q_heads % num_kv_heads != 0:
        raise ValueError("query heads must be a multiple of KV heads")
    S, MB = block_tables.shape
    owner = {}
    for b in range(S):
        T = int(context_lens[b])
        if T < 0 or T > MB * block_size:
            raise ValueError(f"sequence {b}: length {T} outside [0, {MB * block_size}]")
        for j in range(math.ceil(T / block_size)):
            blk = int(block_tables[b, j])
            if not 0 <= blk < num_blocks:
                raise ValueError(f"sequence {b}: block {blk} outside the pool")
            if blk in owner:
                raise ValueError(f"block {blk} used by {owner[blk]} and {(b, j)}")
            owner[blk] = (b, j)


def paged_attention_decode(pool: np.ndarray, dtype: str, layer: int,
                           block_tables: np.ndarray, context_lens: np.ndarray,
                           q: np.ndarray, scale: float, seqs=None) -> np.ndarray:
    """Gather-then-attend, float64, for the sequences in ``seqs`` (default:
    all).  Returns [S, Hq, D]; rows of sequences not in ``seqs`` stay zero.

    The scale is rounded to float32 first, as a float32 argument is what the
    GPU receives.  Sources: see :func:`gather_sequence` and :func:`attend`.
    """
    S, Hq, D = q.shape
    validate_decode_inputs(pool.shape[0], pool.shape[4], block_tables, context_lens, Hq,
                           pool.shape[3])
    scale64 = float(np.float32(scale))
    out = np.zeros((S, Hq, D), dtype=np.float64)
    for b in (range(S) if seqs is None else seqs):
        K, V = gather_sequence(pool, layer, block_tables[b], int(context_lens[b]))
        out[b] = attend(widen(q[b], dtype), widen(K, dtype), widen(V, dtype), scale64)
    return out


def dense_masked_decode(k: np.ndarray, v: np.ndarray, mask: np.ndarray, q: np.ndarray,
                        dtype: str, scale: float, seqs=None) -> np.ndarray:
    """Attention over gathered, padded K/V: k and v are [S, max_len, Hkv, D]
    as the batched gather returns them, mask [S, max_len] marks the cached
    tokens; every position whose mask is 0 is left out of the softmax.
    Returns [S, Hq, D] float64 (rows of sequences not in ``seqs`` stay zero;
    a sequence with no unmasked position gives zeros).

    [mini-infer] "Zero-Copy Batched Attention Gather": the gathered batch is
    the input of the attention for all active sequences at once; the mask
    tells the cached tokens from the padding.
    """
    S, Hq, D = q.shape
    scale64 = float(np.float32(scale))
    out = np.zeros((S, Hq, D), dtype=np.float64)
    for b in (range(S) if seqs is None else seqs):
        keep = np.nonzero(np.asarray(mask[b]) != 0)[0]
        out[b] = attend(widen(q[b], dtype), widen(k[b][keep], dtype), widen(v[b][keep], dtype),
                        scale64)
    return out


# ----------------------------------------------------------------------------
# Memory waste ([mini-infer] "The Problem" and "Memory Waste Analysis")
# ----------------------------------------------------------------------------

def paged_waste_slots(n_tokens: int, block_size: int) -> int:
    """Reserved-but-unused token slots of one sequence under paging: only the
    final block can be partly filled, so waste = ceil(N/B)*B - N."""
    return math.ceil(n_tokens / block_size) * block_size - n_tokens


def paged_waste_ratio(n_tokens: int, block_size: int) -> float:
    """Wasted slots relative to the N tokens held."""
    return paged_waste_slots(n_tokens, block_size) / n_tokens


def paged_waste_bound(n_tokens: int, block_size: int) -> float:
    """The page's closed-form maximum, (B - 1) / N."""
    return (block_size - 1) / n_tokens


def naive_waste_ratio(n_tokens: int, reserved: int) -> float:
    """Contiguous preallocation of ``reserved`` slots holding N tokens."""
    return (reserved - n_tokens) / reserved


# ----------------------------------------------------------------------------
# Free-block stack ([mini-infer] "Python Implementation: Physical Block Pool")
# ----------------------------------------------------------------------------

class OutOfBlocks(MemoryError):
    """The pool has no free physical block left."""


class FreeBlockStack:
    """The page's allocator semantics: every id 0..N-1 starts free in
    ascending order; allocation hands out the most recently pushed id (the
    top of the stack, so N-1 first); freeing pushes the id back.  The page
    performs no check on free; this model does not either."""

    def __init__(self, num_blocks: int):
        self._stack = np.arange(num_blocks, dtype=np.int64)
        self._top = num_blocks          # number of ids currently on the stack

    def __len__(self) -> int:
        return self._top

    def allocate(self) -> int:
        if self._top == 0:
            raise OutOfBlocks("no free block left in the pool")
        self._top -= 1
        return int(self._stack[self._top])

    def free(self, block_id: int) -> None:
        if self._top == len(self._stack):
            self._stack = np.concatenate([self._stack, np.zeros(len(self._stack) + 1, np.int64)])
        self._stack[self._top] = block_id
        self._top += 1
