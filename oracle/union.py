"""Union of the experts selected over a verify's rows.

"Function forward_moe" rustdoc, "RETRACTED (2026-08-29)" note: the
top_k * rows <= 64 selected ids are deduplicated in one block by a pairwise
scan, with no sort, and each expert of the union is then swept once;
"WIDENED (2026-08-31)" note: rows <= 8, so 8 * 8 = 64 ids fill the block.

Definition used here (a reading: the pages give no order).  Flatten the ids
row-major, t = r * k + j.  Slot t is a *first occurrence* when no earlier slot
t' < t holds the same id.  The union lists first occurrences in slot order;
``slot_to_union[t]`` is the union position of slot t's id; bit r of
``row_mask[u]`` is set when row r selected union expert u.

Pinned by tests/test_oracle_union.py against ``dict.fromkeys`` (insertion-
ordered dedup) and ``set`` on exhaustive tiny inputs, and by the bounds
k <= U <= min(k * rows, E).
"""

from __future__ import annotations

from typing import Tuple

import numpy as np


def expert_union(ids: np.ndarray) -> Tuple[np.ndarray, int, np.ndarray, np.ndarray]:
    """ids int [R, k] -> (union_ids int32 [U], U, slot_to_union int32 [R*k], row_mask uint32 [U])."""
    ids = np.asarray(ids)
    R, k = ids.shape
    flat = [int(v) for v in ids.reshape(-1)]
    n = len(flat)
    union_ids = []
    slot_to_union = [0] * n
    for t in range(n):
        first = t
        for t2 in range(t):  # pairwise scan over the earlier slots
            if flat[t2] == flat[t]:
                first = t2
                break
        if first == t:
            slot_to_union[t] = len(union_ids)
            union_ids.append(flat[t])
        else:
            slot_to_union[t] = slot_to_union[first]
    U = len(union_ids)
    row_mask = [0] * U
    for t in range(n):
        row_mask[slot_to_union[t]] |= 1 << (t // k)
    return (np.array(union_ids, dtype=np.int32), U,
            np.array(slot_to_union, dtype=np.int32), np.array(row_mask, dtype=np.uint32))


def expert_union_local(ids: np.ndarray, lo: int, hi: int) -> Tuple[np.ndarray, int, np.ndarray, np.ndarray]:
    """The union of the selected experts that lie in [lo, hi): one GPU's share
    under expert parallelism.

    ``forward_ep.rs`` (``MoeLayer::forward_ep_dispatch``) splits a token's
    selected ids into local and remote ones with ``local_expert_range`` and
    ``build_ep_routing_table``; the rank sweeps only its local experts.  Here:
    slots whose id is outside [lo, hi) are skipped (``slot_to_union[t] = -1``);
    the others form the union exactly as in ``expert_union`` (first occurrence
    in row-major slot order among the local slots).
    """
    ids = np.asarray(ids)
    R, k = ids.shape
    flat = [int(v) for v in ids.reshape(-1)]
    union_ids = []
    slot_to_union = [-1] * len(flat)
    for t, e in enumerate(flat):
        if not (lo <= e < hi):
            continue
        earlier = [t2 for t2 in range(t) if flat[t2] == e]
        if earlier:
            slot_to_union[t] = slot_to_union[earlier[0]]
        else:
            slot_to_union[t] = len(union_ids)
            union_ids.append(e)
    U = len(union_ids)
    row_mask = [0] * U
    for t, u in enumerate(slot_to_union):
        if u >= 0:
            row_mask[u] |= 1 << (t // k)
    return (np.array(union_ids, dtype=np.int32), U,
            np.array(slot_to_union, dtype=np.int32), np.array(row_mask, dtype=np.uint32))
