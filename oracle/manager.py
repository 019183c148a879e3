"""Host block manager model: which physical blocks each sequence holds, and
how many tokens.  TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix:

- Blocks are handed out one at a time as a sequence grows, so only the last
  block of a sequence can be partly filled ([kv-cache] section 2, "Zero-Waste
  Allocation"; [mini-infer] "Memory Waste Analysis").
- Before a step runs, the pool must hold enough free blocks for that step
  ([kv-cache] section 3.1, "Cache Block Pool").
- Blocks come from and go back to one LIFO free stack ([mini-infer] "Python
  Implementation: Physical Block Pool"): ``FreeBlockStack`` here.

Readings where the pages are silent:

- A step either gets every block it needs or nothing changes (all or
  nothing); the error is the pool's out-of-blocks error.
- Within a step, sequences are served in the order given, and each
  sequence's new blocks in logical order.
- A finished sequence returns its blocks in logical order (block 0 first,
  so its last block is the next one handed out).
- A sequence may not grow past ``max_blocks_per_seq`` blocks (the width of
  the block-table rows); that is an argument error, not an out-of-blocks one.
"""

from __future__ import annotations

import math

import numpy as np

from .paged import FreeBlockStack, OutOfBlocks


class BlockManagerModel:
    def __init__(self, num_blocks: int, block_size: int, max_blocks_per_seq: int):
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.max_blocks_per_seq = max_blocks_per_seq
        self.stack = FreeBlockStack(num_blocks)
        self.tables: dict[int, list[int]] = {}
        self.lens: dict[int, int] = {}

    def blocks_for(self, n_tokens: int) -> int:
        """Blocks that hold n tokens: every block full except possibly the last."""
        return math.ceil(n_tokens / self.block_size)

    def add_sequence(self, seq: int) -> None:
        if seq in self.lens:
            raise ValueError(f"sequence {seq} exists")
        self.tables[seq] = []
        self.lens[seq] = 0

    def _check_step(self, seqs, counts) -> int:
        if len(set(seqs)) != len(seqs):
            raise ValueError("a sequence appears twice in one step")
        need = 0
        for s, c in zip(seqs, counts):
            if s not in self.lens or c < 0:
                raise ValueError(f"bad sequence {s} or count {c}")
            after = self.blocks_for(self.lens[s] + c)
            if after > self.max_blocks_per_seq:
                raise ValueError(f"sequence {s} would need {after} blocks")
            need += after - len(self.tables[s])
        return need

    def blocks_needed(self, seqs, counts) -> int:
        """The admission figure: free blocks this step needs."""
        return self._check_step(list(seqs), list(counts))

    def reserve(self, seqs, counts) -> list[int]:
        """Grow sequence seqs[i] by counts[i] tokens; return each one's first
        new position.  Out of blocks: raise, and change nothing."""
        seqs, counts = list(seqs), list(counts)
        need = self._check_step(seqs, counts)
        if need > len(self.stack):
            raise OutOfBlocks("no free block left in the pool")
        starts = []
        for s, c in zip(seqs, counts):
            while len(self.tables[s]) < self.blocks_for(self.lens[s] + c):
                self.tables[s].append(self.stack.allocate())
            starts.append(self.lens[s])
            self.lens[s] += c
        return starts

    def release(self, seq: int) -> None:
        for blk in self.tables.pop(seq):
            self.stack.free(blk)
        del self.lens[seq]

    def block_tables(self, seqs) -> tuple[np.ndarray, np.ndarray]:
        """int32 [n, max_blocks_per_seq] rows (-1 past the used blocks) and
        int32 [n] token counts."""
        seqs = list(seqs)
        tab = np.full((len(seqs), self.max_blocks_per_seq), -1, dtype=np.int32)
        lens = np.zeros(len(seqs), dtype=np.int32)
        for i, s in enumerate(seqs):
            tab[i, :len(self.tables[s])] = self.tables[s]
            lens[i] = self.lens[s]
        return tab, lens

    def stats(self) -> dict:
        used = sum(len(t) for t in self.tables.values())
        tokens = sum(self.lens.values())
        slots = used * self.block_size
        return dict(sequences=len(self.lens), blocks_total=self.num_blocks,
                    blocks_free=len(self.stack), blocks_used=used, tokens=tokens,
                    slots=slots, waste_slots=slots - tokens,
                    waste_ratio=(slots - tokens) / tokens if tokens else 0.0)
