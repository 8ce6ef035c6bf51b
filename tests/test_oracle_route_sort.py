"""Pins of the oracle's specified exp/sigmoid, routing and sorting: exact special
values, float64 error bounds, definition checks on every token, exhaustive
group-subset enumeration, closed-form weights, torch.topk, and an independent
stable argsort."""

import itertools

import numpy as np
import pytest
import torch

import oracle
from oracle.specmath import CLAMP


def _ulp_err(got32, ref64):
    got = got32.astype(np.float64)
    ulp = np.spacing(np.abs(ref64).astype(np.float32)).astype(np.float64)
    return np.abs(got - ref64) / ulp


def test_spec_exp_special_values():
    assert oracle.spec_exp(np.float32(0.0)) == np.float32(1.0)
    assert oracle.spec_sigmoid(np.float32(0.0)) == np.float32(0.5)
    assert oracle.spec_exp(np.float32(1000.0)) == oracle.spec_exp(CLAMP)
    assert oracle.spec_exp(np.float32(-1000.0)) == oracle.spec_exp(-CLAMP)
    assert oracle.spec_sigmoid(np.float32(200.0)) == np.float32(1.0)


def test_spec_exp_within_two_ulp():
    x = np.linspace(-80, 80, 2_000_001).astype(np.float32)
    err = _ulp_err(oracle.spec_exp(x), np.exp(x.astype(np.float64)))
    assert err.max() <= 2.0, err.max()


def test_spec_sigmoid_within_three_ulp_and_monotone():
    x = np.linspace(-80, 80, 2_000_001).astype(np.float32)
    s = oracle.spec_sigmoid(x)
    ref = 1.0 / (1.0 + np.exp(-x.astype(np.float64)))
    # exp within 2 ulp, then one rounded add (<= 0.5 ulp of 1+e) and one rounded
    # division (0.5 ulp): at most 3 ulp in total
    assert _ulp_err(s, ref).max() <= 3.0
    assert np.all(np.diff(s.astype(np.float64)) >= 0)


def _check_selection(keys, ids, k, eligible):
    """Definition of top-k with the tie rule: every selected expert beats every
    unselected eligible one (larger key, or equal key and lower index), and the
    ids come in rank order."""
    sel = list(ids)
    assert len(set(sel)) == k
    rest = [e for e in eligible if e not in sel]
    for a in sel:
        for b in rest:
            assert keys[a] > keys[b] or (keys[a] == keys[b] and a < b)
    for a, b in zip(sel, sel[1:]):
        assert keys[a] > keys[b] or (keys[a] == keys[b] and a < b)


def test_softmax_route_definition_and_weights():
    rng = np.random.default_rng(5)
    T, E, k = 64, 32, 6
    logits = rng.normal(0, 1, (T, E)).astype(np.float32)
    ids, w = oracle.route(logits, topk=k, routed_scaling_factor=1.7)
    for t in range(T):
        _check_selection(logits[t], ids[t], k, range(E))
        p = np.exp(logits[t].astype(np.float64))
        ref = p[ids[t]] / p[ids[t]].sum() * 1.7
        assert np.allclose(w[t], ref, rtol=1e-14, atol=0)
        assert abs(w[t].sum() - 1.7) <= 1e-14


def test_softmax_route_matches_torch_topk_without_ties():
    rng = np.random.default_rng(6)
    logits = rng.normal(0, 1, (200, 64)).astype(np.float32)
    ids, _ = oracle.route(logits, topk=8)
    ref = torch.topk(torch.from_numpy(logits), 8, dim=1).indices.numpy()
    assert np.array_equal(ids, ref)


def test_tie_heavy_logits():
    rng = np.random.default_rng(7)
    logits = rng.integers(-1, 2, (100, 16)).astype(np.float32)
    ids, _ = oracle.route(logits, topk=5)
    for t in range(100):
        order = sorted(range(16), key=lambda e: (-logits[t, e], e))
        assert list(ids[t]) == order[:5]
    sids, _ = oracle.route(logits, topk=5, score="sigmoid")
    assert np.array_equal(sids, ids)  # sigmoid is monotone and equal logits tie


def test_equal_logits_closed_form():
    for score in ("softmax", "sigmoid"):
        ids, w = oracle.route(np.zeros((3, 16), np.float32), topk=8, score=score, routed_scaling_factor=2.5)
        assert np.array_equal(ids, np.tile(np.arange(8), (3, 1)))
        assert np.all(w == 0.3125)


def test_k_equals_e_softmax_is_scaled_softmax():
    rng = np.random.default_rng(8)
    logits = rng.normal(0, 2, (10, 8)).astype(np.float32)
    ids, w = oracle.route(logits, topk=8, routed_scaling_factor=3.0)
    sm = torch.softmax(torch.from_numpy(logits).double(), dim=1).numpy()
    for t in range(10):
        assert np.allclose(w[t], sm[t, ids[t]] * 3.0, rtol=1e-13)


def test_no_renormalize():
    rng = np.random.default_rng(9)
    logits = rng.normal(0, 1, (10, 8)).astype(np.float32)
    ids, w = oracle.route(logits, topk=3, renormalize=False, score="sigmoid")
    assert np.allclose(w, 1.0 / (1.0 + np.exp(-logits.astype(np.float64)[np.arange(10)[:, None], ids])))


def test_grouped_selection_exhaustive_subsets():
    rng = np.random.default_rng(10)
    E, G, Gk, k = 16, 4, 2, 3
    eg = E // G
    for trial in range(60):
        logits = rng.normal(0, 1, (1, E)).astype(np.float32)
        if trial % 3 == 0:
            logits = rng.integers(-1, 2, (1, E)).astype(np.float32)  # ties
        bias = (rng.normal(0, 0.1, E)).astype(np.float32)
        ids, _ = oracle.route(logits, topk=k, score="sigmoid", bias=bias, n_group=G, topk_group=Gk)
        c = (oracle.spec_sigmoid(logits[0]) + bias).astype(np.float32)
        gs = []
        for g in range(G):
            top = sorted(c[g * eg:(g + 1) * eg], reverse=True)
            gs.append(np.float32(top[0]) + np.float32(top[1]))
        winners = []
        for S in itertools.combinations(range(G), Gk):
            if all(gs[a] > gs[b] or (gs[a] == gs[b] and a < b) for a in S for b in range(G) if b not in S):
                winners.append(S)
        assert len(winners) == 1
        eligible = [e for e in range(E) if e // eg in winners[0]]
        _check_selection(c, ids[0], k, eligible)


def test_group_score_top1_variant():
    logits = np.array([[5, -9, -9, -9, 1, 1, -9, -9]], np.float32)
    ids2, _ = oracle.route(logits, topk=2, score="sigmoid", n_group=2, topk_group=1, group_score_topk=2)
    ids1, _ = oracle.route(logits, topk=2, score="sigmoid", n_group=2, topk_group=1, group_score_topk=1)
    assert list(ids2[0]) == [4, 5]   # sigma(1)+sigma(1) > sigma(5)+sigma(-9)
    assert list(ids1[0]) == [0, 1]   # max: sigma(5) wins


def test_pseudo_slots():
    ids, w = oracle.route(np.zeros((4, 8), np.float32), topk=2, n_pseudo=3, gamma=np.array([0.1, 0.2, 0.3, 0.4]))
    assert np.array_equal(ids[:, 2:], np.tile([8, 9, 10], (4, 1)))
    assert np.allclose(w[:, 2:], np.array([0.1, 0.2, 0.3, 0.4])[:, None])


@pytest.mark.parametrize("block_m", [1, 4, 16, 64])
def test_sort_against_stable_argsort(block_m):
    rng = np.random.default_rng(11)
    T, k, E = 50, 4, 12
    # distinct experts per token, expert 7 never chosen (an empty expert)
    ids = np.stack([rng.choice([e for e in range(E) if e != 7], k, replace=False) for _ in range(T)]).astype(np.int32)
    r = oracle.sort_tokens(ids, E, block_m)
    flat = ids.reshape(-1)
    order = np.argsort(flat, kind="stable")
    P = flat.size
    expect = []
    be = []
    for e in range(E):
        mine = order[flat[order] == e]
        pad = -(-len(mine) // block_m) * block_m
        expect += list(mine) + [P] * (pad - len(mine))
        be += [e] * (pad // block_m)
    assert np.array_equal(r["sorted_pair_ids"], np.array(expect))
    assert np.array_equal(r["block_expert"], np.array(be))
    assert r["counts"].sum() == P and r["counts"][7] == 0
    assert r["num_blocks"] == len(be) and r["offsets"][-1] == len(expect)
    real = r["sorted_pair_ids"][r["sorted_pair_ids"] < P]
    assert np.array_equal(np.sort(real), np.arange(P))
