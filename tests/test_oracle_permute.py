"""Pins of the oracle's permute map (expanded_idx_to_permuted_idx of the
output-contract page: int32 [num_tokens, top_k], -1 for an expert that is not
local; per-local-expert counts of the modular-kernel page's prepare).

Pins: a hand-worked example, the structural invariants (bijection onto the
local rows, count sum, segment membership, stable order) and equality with a
stable numpy argsort of the local expert ids over the expanded index."""
import numpy as np
import pytest

import oracle
import synth
from synth import configs


def test_hand_worked_example():
    ids = np.array([[1, 0], [0, 1], [1, 2]], dtype=np.int32)
    m, off, cnt = oracle.permute(ids, E=3, E_l=3)
    assert cnt.tolist() == [2, 3, 1]
    assert off.tolist() == [0, 2, 5, 6]
    assert m.tolist() == [[2, 0], [1, 3], [4, 5]]


def test_hand_worked_example_with_map():
    ids = np.array([[3, 0], [1, 3], [2, 0]], dtype=np.int32)
    emap = np.array([-1, 1, -1, 0], dtype=np.int32)     # experts 3 -> 0, 1 -> 1 local
    m, off, cnt = oracle.permute(ids, E=4, E_l=2, expert_map=emap)
    assert cnt.tolist() == [2, 1]
    assert off.tolist() == [0, 2, 3]
    assert m.tolist() == [[0, -1], [2, 1], [-1, -1]]


def _random_ids(seed, T, E, k):
    logits = synth.normal_f32(seed, 1, (T, E))
    ids, _ = oracle.route(logits, k, oracle.SOFTMAX, True, 1.0)
    return ids


def _check_invariants(ids, emap, E, E_l):
    m, off, cnt = oracle.permute(ids, E=E, E_l=E_l, expert_map=emap)
    T, k = ids.shape
    L = ids if emap is None else emap[ids]
    nonlocal_ = int(np.sum(L < 0))
    R_l = T * k - nonlocal_
    # counts sum to the local routes, offsets are their exclusive scan
    assert cnt.sum() == R_l
    assert off[0] == 0 and np.array_equal(np.diff(off), cnt)
    # -1 exactly where the expert is not local
    assert np.array_equal(m < 0, L < 0) and np.all(m[m < 0] == -1)
    # bijection onto [0, R_l)
    assert np.array_equal(np.sort(m[m >= 0]), np.arange(R_l))
    # each route lands in its expert's segment, in increasing token order
    for e in range(E_l):
        t_idx, j_idx = np.nonzero(L == e)
        rows = m[t_idx, j_idx]
        assert np.all((rows >= off[e]) & (rows < off[e + 1]))
        assert np.all(np.diff(rows[np.argsort(t_idx * k + j_idx)]) == 1)
    # equals a stable argsort of the local ids over the expanded index
    flat = L.reshape(-1)
    keep = np.nonzero(flat >= 0)[0]
    order = keep[np.argsort(flat[keep], kind="stable")]
    inv = np.full(T * k, -1, dtype=np.int64)
    inv[order] = np.arange(order.size)
    assert np.array_equal(m.reshape(-1), inv)
    return m, off


@pytest.mark.parametrize("T,E,k", [(16, 8, 2), (300, 8, 2), (200, 256, 8), (9, 4, 4)])
def test_invariants_all_local(T, E, k):
    _check_invariants(_random_ids(31 + T, T, E, k), None, E, E)


@pytest.mark.parametrize("T", [1, 8, 64, 500])
def test_invariants_ep_rank_map(T):
    cfg = configs.EP_DECODE
    ids = _random_ids(41 + T, T, cfg.E, cfg.k)
    _check_invariants(ids, configs.expert_map(cfg), cfg.E, cfg.El)


def test_scattered_map():
    E, E_l = 64, 10
    rng = np.random.default_rng(5)
    emap = np.full(E, -1, dtype=np.int32)
    emap[rng.choice(E, E_l, replace=False)] = rng.permutation(E_l)
    _check_invariants(_random_ids(51, 128, E, 6), emap, E, E_l)


def test_all_routes_nonlocal():
    ids = np.array([[0, 1], [1, 0]], dtype=np.int32)
    emap = np.array([-1, -1, 0], dtype=np.int32)
    m, off, cnt = oracle.permute(ids, E=3, E_l=1, expert_map=emap)
    assert np.all(m == -1) and off.tolist() == [0, 0] and cnt.tolist() == [0]


def test_empty_input():
    ids = np.zeros((0, 8), dtype=np.int32)
    m, off, cnt = oracle.permute(ids, E=256, E_l=256)
    assert m.shape == (0, 8) and np.all(off == 0)


def test_out_of_range_id_rejected():
    with pytest.raises(ValueError):
        oracle.permute(np.array([[0, 5]], dtype=np.int32), E=4, E_l=4)
