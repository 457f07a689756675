"""Oracle: longest-processing-time-first chunk assignment with equal chunk counts.

Test infrastructure only; never used by the product path.

Split-KV's planner visits context chunks from the most to the least costly and
puts each on the device with the least work so far among those that still have
room, so that every device ends with the same number of chunks ("Split-KV speeds diffusion drafter training...", section
"Balance actual attention work").  Readings taken where the page is silent:

* eligible = holding fewer than n_chunk / n_bin chunks (n_chunk must be a
  multiple of n_bin, otherwise equal counts are impossible);
* chunks are visited by (cost descending, chunk index ascending) and the bin is
  the eligible one with the smallest (load, bin index), which makes the plan
  unique so that every device derives the same plan from the same costs;
* imbalance = max load / mean load - 1.
"""

from __future__ import annotations


def lpt_assign(cost, n_bin: int):
    """Returns (bin_of_chunk list[int], bin_load list[int])."""
    cost = [int(c) for c in cost]
    n = len(cost)
    if n_bin <= 0 or n % n_bin != 0:
        raise ValueError("chunk count must be a positive multiple of the bin count")
    cap = n // n_bin
    order = sorted(range(n), key=lambda c: (-cost[c], c))
    load = [0] * n_bin
    count = [0] * n_bin
    bin_of = [-1] * n
    for c in order:
        best = None
        for b in range(n_bin):
            if count[b] >= cap:
                continue
            if best is None or (load[b], b) < (load[best], best):
                best = b
        bin_of[c] = best
        load[best] += cost[c]
        count[best] += 1
    return bin_of, load


def imbalance(load) -> float:
    load = [int(x) for x in load]
    mean = sum(load) / len(load)
    return max(load) / mean - 1.0 if mean > 0 else 0.0
