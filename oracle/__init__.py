"""CPU oracle for paged-KV-cache attention decode.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import, call or run anything in
this package.  The product path (the HIP library and its Python binding)
never touches it, and it shares no code with that path: the only common
dependency is the seeded input generator package ``workloads``.

Everything here is plain, slow and meant to be checked by eye against the
pages it cites.  Floating point is float64.  Pins (tests/test_oracle_*.py)
tie each function to something other than itself.

Parity status per function:
  logical_to_physical, resolve_slots   pinned (page examples, invariants)
  gather_sequence, paged_kv_gather     pinned (page examples, coordinate-
                                       encoded pool, contiguous equivalence)
  kv_append                            pinned (hand-derived fixture,
                                       whole-pool diff, gather round trip)
  kv_append_layers, kv_append_tokens   pinned (hand-derived fixtures; equal
                                       to per-layer / per-token kv_append)
  attend, paged_attention_decode       pinned (torch SDPA in float64,
                                       brute force, closed forms, invariants)
  dense_masked_decode                  pinned (equal to the paged decode on
                                       the gathered batch; brute force with
                                       random masks; masked rows ignored)
  waste arithmetic                     pinned (the page's worked numbers)
  FreeBlockStack                       pinned (the page's LIFO semantics)
  BlockManagerModel (manager.py)       pinned (the pages' waste figures and
                                       bound, LIFO reuse, all-or-nothing
                                       admission, conservation of blocks)
"""

from .manager import BlockManagerModel  # noqa: F401
from .paged import (  # noqa: F401
    FreeBlockStack,
    OutOfBlocks,
    attend,
    dense_masked_decode,
    gather_sequence,
    kv_append,
    kv_append_layers,
    kv_append_tokens,
    kv_head_of,
    logical_to_physical,
    naive_waste_ratio,
    paged_attention_decode,
    paged_kv_gather,
    paged_waste_bound,
    paged_waste_ratio,
    paged_waste_slots,
    resolve_slots,
    validate_decode_inputs,
    widen,
)
