"""Top-k routing, written from the pages' description, one token at a time.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

What the pages fix:

* The router produces top-k expert ids and top-k weights per token, and the
  routed scaling factor is folded into those weights instead of multiplying the
  MoE output (vLLM PR 65207, Purpose, commit 1: AITER's biased grouped top-k
  applies it in-kernel).  The shared expert is never scaled by it.
* Sigmoid scoring with a per-expert bias and expert groups ("biased grouped
  top-k", same passage).

Readings where the pages are silent (each is listed in the design notes):

* softmax scoring ranks experts by logit (softmax is monotone, so this is the
  same order, computed exactly); weights are softmax probabilities over all E,
  renormalised over the k selected when ``renormalize``;
* sigmoid scoring selects on sigmoid(logit) + bias, with sigmoid computed by
  the fully specified float32 routine of ``specmath`` so that the decision is
  reproducible; the weights use the unbiased sigmoid (float64 here);
* groups are ``n_group`` blocks of E / n_group consecutive experts; a group's
  score is the sum of its two largest biased scores (``group_score_topk=2``)
  or its largest (``=1``), summed in float32; the ``topk_group`` best groups are
  kept and the top-k is taken among their experts;
* ties: the larger score wins, equal scores go to the lower index (expert or
  group); ids are emitted in rank order;
* ``routed_scaling_factor`` multiplies the weights after renormalisation;
* optional shared pseudo-expert slots ``E .. E+n_pseudo-1`` are appended with
  the shared gate value as their weight (the heterogeneous fused layer of vLLM
  PR 61503, Overview, treats the shared expert as always selected).
"""

import numpy as np

from .specmath import spec_sigmoid


def _rank_desc(keys, idx):
    """Indices ``idx`` ordered by ``keys`` descending, ties to the lower index."""
    keys = np.asarray(keys)
    idx = np.asarray(idx)
    order = np.lexsort((idx, -keys.astype(np.float64)))
    return idx[order]


def route(logits, *, topk, score="softmax", bias=None, n_group=1, topk_group=1,
          group_score_topk=2, renormalize=True, routed_scaling_factor=1.0,
          n_pseudo=0, gamma=None):
    """Route every token.

    logits: float32 [T, E].  bias: float32 [E] or None (sigmoid scoring only).
    Returns (ids int32 [T, topk + n_pseudo], weights float64 [T, topk + n_pseudo]).
    """
    logits = np.asarray(logits, dtype=np.float32)
    T, E = logits.shape
    if bias is None:
        bias = np.zeros(E, dtype=np.float32)
    bias = np.asarray(bias, dtype=np.float32)
    ids = np.zeros((T, topk + n_pseudo), dtype=np.int32)
    w = np.zeros((T, topk + n_pseudo), dtype=np.float64)
    experts = np.arange(E)
    for t in range(T):
        lt = logits[t]
        if score == "softmax":
            key = lt
        elif score == "sigmoid":
            key = (spec_sigmoid(lt) + bias).astype(np.float32)
        else:
            raise ValueError(score)

        eligible = experts
        if n_group > 1:
            eg = E // n_group
            gscore = np.zeros(n_group, dtype=np.float32)
            for g in range(n_group):
                top = np.sort(key[g * eg:(g + 1) * eg])[::-1]
                if group_score_topk == 2:
                    gscore[g] = np.float32(top[0]) + np.float32(top[1])
                else:
                    gscore[g] = top[0]
            kept = _rank_desc(gscore, np.arange(n_group))[:topk_group]
            eligible = np.sort(np.concatenate([np.arange(g * eg, (g + 1) * eg) for g in kept]))

        sel = _rank_desc(key[eligible], eligible)[:topk]
        ids[t, :topk] = sel

        l64 = lt.astype(np.float64)
        if score == "softmax":
            p = np.exp(l64 - l64.max())
            p = p / p.sum()
        else:
            p = 1.0 / (1.0 + np.exp(-l64))
        ws = p[sel]
        if renormalize:
            ws = ws / ws.sum()
        w[t, :topk] = ws * routed_scaling_factor

        for j in range(n_pseudo):
            ids[t, topk + j] = E + j
            w[t, topk + j] = 1.0 if gamma is None else float(gamma[t])
    return ids, w
