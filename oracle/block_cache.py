"""LRU cache of selected blocks and the step difference (CPU oracle).

TEST INFRASTRUCTURE ONLY, like the rest of this package: the library never
uses it.

Follows "SGLang hierarchical sparse attention: analysis and practice",
section 3.2 (the sparse diff kernel): consecutive decode steps select largely
the same blocks, so the GPU keeps a cache pool a few times larger than the
top-k, managed least-recently-used; each step (a) takes the difference
between this step's selection and the previous one, (b) finds the blocks
already cached (hits), (c) would load the misses, and (d) updates the cache
index. Without a host tier, the cache here is its index alone.

Readings (the page gives the policy, not the bookkeeping):
  * a unit's cache is `capacity` slots, each holding a block id (-1 = empty)
    and the step at which that block was last selected (-1 for empty slots);
  * at step t every selected block that is cached is a hit and its stamp
    becomes t; the misses, in ascending block order, take the slots not hit at
    this step in order of (stamp ascending, slot index ascending) -- empty
    slots first, then least recently used -- and get stamp t;
  * the step difference is |S_t minus S_(t-1)|: selected blocks whose slot did
    not carry stamp t - 1. With capacity >= |S_(t-1)| + |S_t| no block of
    S_(t-1) can have been evicted before step t, so this equals the set
    difference (the pages' "2-4 x top-k" pool satisfies that).
Plain Python loops: capacities and selections are at most a few thousand.
"""
from __future__ import annotations

from typing import List, Sequence, Tuple


def cache_step(slot_block: Sequence[int], slot_stamp: Sequence[int], ids: Sequence[int],
               step: int) -> Tuple[List[int], List[int], List[int], List[int], int, int, int]:
    """One step of one unit. ids: this step's selection, ascending, distinct.
    Returns (new slot_block, new slot_stamp, slot of each selected block,
    missed blocks in ascending order, hits, misses, step difference)."""
    blk = [int(x) for x in slot_block]
    st = [int(x) for x in slot_stamp]
    cap = len(blk)
    if len(ids) > cap:
        raise ValueError("selection larger than the cache")
    where = {b: s for s, b in enumerate(blk) if b >= 0}
    hit = [False] * cap
    slot_of = [-1] * len(ids)
    missed_j = []
    still_there = 0  # selected blocks that were selected at step - 1 too
    for j, b in enumerate(ids):
        s = where.get(int(b))
        if s is None:
            missed_j.append(j)
            continue
        if st[s] == step - 1:
            still_there += 1
        st[s] = step
        hit[s] = True
        slot_of[j] = s
    victims = sorted((st[s], s) for s in range(cap) if not hit[s])
    for r, j in enumerate(missed_j):
        s = victims[r][1]
        blk[s] = int(ids[j])
        st[s] = step
        slot_of[j] = s
    misses = [int(ids[j]) for j in missed_j]
    return (blk, st, slot_of, misses, len(ids) - len(missed_j), len(missed_j),
            len(ids) - still_there)
