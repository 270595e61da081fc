"""Routing of the oracle: top-k expand, histogram, offsets, stable permutation.

Definition (HyperMegaMoE RFC, section 4.1 "routing and expert parallel"; the
usage guide, "inputs and weights"; MoeDistributeDispatchV2 parameter table,
expertTokenNums):

* every token t is expanded into K expert slots; slot s = t*K + k carries the
  global expert id ``topk_ids[t, k]``;
* ``counts[e]`` is the exact number of slots routed to expert e (the per-expert
  token histogram, int32);
* ``offsets`` is the exclusive prefix sum of ``counts`` with ``offsets[E]`` =
  T*K (the RFC's offset construction; the dispatch op's prefix-sum form of the
  expert token numbers is ``offsets[1:]``);
* the slots are sorted by expert (RFC section 6.2 names sorting by expert and
  the reverse un-sort).  The pages do not order slots of one expert; the
  reading here is the stable one: ascending slot index inside each expert.
  ``sorted_slot[p]`` is the slot placed at permuted row p and
  ``row_of_slot[s]`` is its inverse.

All results are int32 and must be reproduced bit for bit.
"""

import numpy as np


def check_ids(topk_ids, E):
    """Raise ValueError if any id lies outside [0, E) (RFC section 4.2)."""
    ids = np.asarray(topk_ids)
    if ids.size and (ids.min() < 0 or ids.max() >= E):
        raise ValueError("topk_ids must lie in [0, E)")


def route(topk_ids, E):
    """Return dict(counts[E], offsets[E+1], sorted_slot[S], row_of_slot[S]), int32.

    Slots are visited in ascending order; each one takes the next free row of
    its expert, which is the stable placement described in the module text.
    """
    check_ids(topk_ids, E)
    ids = np.asarray(topk_ids, dtype=np.int64).reshape(-1)
    S = ids.size
    counts = np.zeros(E, dtype=np.int64)
    for e in ids:
        counts[e] += 1
    offsets = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]
    next_row = offsets[:E].copy()
    row_of_slot = np.empty(S, dtype=np.int64)
    sorted_slot = np.empty(S, dtype=np.int64)
    for s in range(S):
        e = ids[s]
        row_of_slot[s] = next_row[e]
        sorted_slot[next_row[e]] = s
        next_row[e] += 1
    return {
        "counts": counts.astype(np.int32),
        "offsets": offsets.astype(np.int32),
        "sorted_slot": sorted_slot.astype(np.int32),
        "row_of_slot": row_of_slot.astype(np.int32),
    }


def permute_rows(rows, sorted_slot, K):
    """Dispatch on one device: permuted row p holds token sorted_slot[p] // K."""
    return np.asarray(rows)[np.asarray(sorted_slot, dtype=np.int64) // K]


def unpermute_rows(prows, row_of_slot):
    """Un-sort: slot s (= t*K + k) receives permuted row row_of_slot[s]."""
    return np.asarray(prows)[np.asarray(row_of_slot, dtype=np.int64)]
