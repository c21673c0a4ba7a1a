"""Layer-parallel set plan.

Source: EasySpec rebuttal, reply on Table 4 (automated strategies) and reply on
Figure 1(b).  The first and the last draft layer are never parallelised; the
intermediate layers are grouped into sets of the layer-parallel size N, and a
trailing set that cannot be filled (because the next layer is the last) stays
smaller.  The worked example for N = 4 and 32 layers ends with the 3-set
{28, 29, 30}.

Reading adopted (the notation on the page is garbled): aligned blocks.  An
intermediate layer l (1 <= l <= L-2) belongs to set floor(l / N); layers 0 and
L-1 are singletons.  This reproduces "N ~ 2N-1", "4 ~ 7", "28 ~ 30" and the
forced 3-set of the worked example.
"""
from __future__ import annotations

from typing import List


def default_group_plan(n_layers: int, group_size: int) -> List[List[int]]:
    if n_layers < 1 or group_size < 1:
        raise ValueError("n_layers and group_size must be >= 1")
    sets: List[List[int]] = [[0]]
    if n_layers == 1:
        return sets
    current_key = None
    for l in range(1, n_layers - 1):
        key = l // group_size
        if key != current_key:
            sets.append([])
            current_key = key
        sets[-1].append(l)
    sets.append([n_layers - 1])
    return sets


def plan_offsets(sets: List[List[int]]) -> List[int]:
    """CSR offsets of a contiguous plan (validated)."""
    offs = [0]
    nxt = 0
    for s in sets:
        if not s or s != list(range(nxt, nxt + len(s))):
            raise ValueError("plan sets must be non-empty, contiguous and in order")
        nxt += len(s)
        offs.append(nxt)
    return offs


def offsets_to_sets(offsets) -> List[List[int]]:
    return [list(range(offsets[i], offsets[i + 1])) for i in range(len(offsets) - 1)]
