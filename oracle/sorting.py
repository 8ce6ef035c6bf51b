"""Token-by-expert sort with per-expert padding, from its definition.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

vLLM PR 65207 (Purpose, commit 2, and the review's experiment with "moe_sorting
without zeroing") names a sorting step that runs before stage 1 but does not
give its layout.  Reading used here: a (token, slot) pair has the flat index
p = t * k_total + slot.  Experts are laid out in index order; within an expert
the pair indices are listed in ascending order; each expert's list is padded up
to a multiple of ``block_m`` with the sentinel value P = T * k_total; an expert
with no pairs gets no block.  ``block_expert[b]`` names the expert that owns
block b.
"""

import numpy as np


def sort_tokens(ids, n_experts, block_m):
    """ids: int [T, k_total] expert ids in [0, n_experts).

    Returns a dict with counts [n_experts], offsets [n_experts + 1] (padded
    exclusive scan), sorted_pair_ids [offsets[-1]], block_expert [num_blocks]
    and num_blocks.
    """
    flat = np.asarray(ids).reshape(-1)
    P = flat.size
    counts = np.zeros(n_experts, dtype=np.int64)
    lists = []
    for e in range(n_experts):
        pairs = np.nonzero(flat == e)[0]          # ascending pair index
        counts[e] = pairs.size
        lists.append(pairs)
    padded = -(-counts // block_m) * block_m
    offsets = np.concatenate([[0], np.cumsum(padded)]).astype(np.int64)
    sorted_ids = np.full(int(offsets[-1]), P, dtype=np.int64)
    block_expert = []
    for e in range(n_experts):
        sorted_ids[offsets[e]:offsets[e] + counts[e]] = lists[e]
        block_expert += [e] * int(padded[e] // block_m)
    return {
        "counts": counts.astype(np.int32),
        "offsets": offsets.astype(np.int32),
        "sorted_pair_ids": sorted_ids.astype(np.int32),
        "block_expert": np.asarray(block_expert, dtype=np.int32),
        "num_blocks": len(block_expert),
    }
