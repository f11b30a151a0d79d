"""Route metadata: per-expert counts, offsets and the stable permutation.

TEST INFRASTRUCTURE ONLY: nothing in the product path may import this module.

A route is one (token t, slot s) pair with flat index f = t*k + s.  Routes whose
expert id lies outside [0, E) (negative, or an expert that is not resident
here) get no row: they contribute an exact zero (b12x PR #339, commit "FC2-only
route validation": invalid ids get an exact-zero effective weight; pegainfer
PR #867, commit 7c19a7a0: expert-windowed metadata, non-local experts skipped).
Within an expert the rows keep ascending f, and experts are laid out in
ascending id order (pegainfer PR #867, commit 53edfa98: "race-free per-expert
compaction, deterministic token*topk+slot entry order").

Two independent formulations are kept so that each pins the other:
``route_sort`` (counting sort, one pass in f order) and ``route_sort_by_key``
(Python's ``sorted`` on the key (expert, f)).

Outputs (all int32):
  counts[E]      rows per expert
  offsets[E+1]   exclusive prefix sum of counts (offsets[E] = R)
  perm[R]        flat route index of each row, rows ordered by (expert, f)
  rowpos[T*k]    row of route f, or -1 for an invalid route
"""
from __future__ import annotations

import numpy as np


def _valid(e: int, experts: int) -> bool:
    return 0 <= e < experts


def route_sort(topk_ids: np.ndarray, experts: int):
    ids = np.asarray(topk_ids, dtype=np.int64).reshape(-1)
    counts = [0] * experts
    for e in ids:
        if _valid(int(e), experts):
            counts[int(e)] += 1
    offsets = [0] * (experts + 1)
    for e in range(experts):
        offsets[e + 1] = offsets[e] + counts[e]
    nxt = offsets[:-1].copy()
    perm = [0] * offsets[experts]
    rowpos = [-1] * ids.size
    for f, e in enumerate(ids):
        e = int(e)
        if _valid(e, experts):
            perm[nxt[e]] = f
            rowpos[f] = nxt[e]
            nxt[e] += 1
    i32 = lambda a: np.asarray(a, dtype=np.int32)
    return i32(counts), i32(offsets), i32(perm), i32(rowpos)


def route_sort_by_key(topk_ids: np.ndarray, experts: int):
    ids = [int(e) for e in np.asarray(topk_ids).reshape(-1)]
    valid = [f for f, e in enumerate(ids) if _valid(e, experts)]
    perm = sorted(valid, key=lambda f: (ids[f], f))
    rowpos = [-1] * len(ids)
    for pos, f in enumerate(perm):
        rowpos[f] = pos
    counts = [sum(1 for f in valid if ids[f] == e) for e in range(experts)] if len(valid) < 4096 \
        else list(np.bincount([ids[f] for f in valid], minlength=experts))
    offsets = [0]
    for c in counts:
        offsets.append(offsets[-1] + int(c))
    i32 = lambda a: np.asarray(a, dtype=np.int32)
    return i32(counts), i32(offsets), i32(perm), i32(rowpos)
