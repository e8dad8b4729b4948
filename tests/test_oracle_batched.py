"""Pins of the oracle's permute into the batched experts format (vLLM
modular_kernel.py: FusedMoEActivationFormat.BatchedExperts, (local experts,
max tokens per expert, hidden), with per-expert token counts from prepare).

- a hand-worked example with a capacity that drops routes;
- with capacity >= T nothing drops, and each route's position inside its
  expert equals its position in the standard (pinned) permute's segment;
- every kept route owns one row of its expert's block, in expanded order;
- routes to experts that are not local get -1.
"""
import numpy as np

import oracle
import synth
from synth import configs


def test_hand_worked_capacity_two():
    ids = np.array([[0, 2], [2, 1], [0, 2], [1, 0]], dtype=np.int32)
    m, counts = oracle.permute_batched(ids, E=3, E_l=3, max_tokens=2)
    # expert 0: x = 0, 4 -> rows 0, 1; x = 7 dropped
    # expert 1: x = 3, 6 -> rows 2, 3
    # expert 2: x = 1, 2 -> rows 4, 5; x = 5 dropped
    want = np.array([[0, 4], [5, 2], [1, -1], [3, -1]], dtype=np.int32)
    assert np.array_equal(m, want)
    assert counts.tolist() == [3, 2, 3]


def test_no_drop_matches_standard_segments():
    T, k, E = 40, 3, 7
    logits = synth.normal_f32(51, 1, (T, E))
    ids, _ = oracle.route(logits, k, configs.SOFTMAX, True, 1.0)
    m_std, off, cnt = oracle.permute(ids, E, E)
    m_b, cnt_b = oracle.permute_batched(ids, E, E, max_tokens=T)
    assert np.array_equal(cnt_b, cnt)
    L = ids  # no expert map: local id = global id
    assert np.array_equal(m_b - L * T, m_std - off[L])


def test_kept_routes_fill_each_block_in_order():
    T, k, E, M = 64, 4, 8, 20
    logits = synth.normal_f32(52, 1, (T, E))
    logits[:, 0] += 3.0  # expert 0 overflows its 20 slots
    ids, _ = oracle.route(logits, k, configs.SOFTMAX, True, 1.0)
    m, counts = oracle.permute_batched(ids, E, E, max_tokens=M)
    assert counts[0] > M
    flat_ids, flat_m = ids.reshape(-1), m.reshape(-1)
    for e in range(E):
        rows = flat_m[(flat_ids == e) & (flat_m >= 0)]
        n = min(int(counts[e]), M)
        assert np.array_equal(rows, e * M + np.arange(n))  # expanded order, no gaps
        assert np.sum((flat_ids == e) & (flat_m < 0)) == int(counts[e]) - n
    kept = flat_m[flat_m >= 0]
    assert len(np.unique(kept)) == len(kept)


def test_nonlocal_routes_get_minus_one():
    ids = np.array([[0, 1], [2, 3], [3, 0]], dtype=np.int32)
    emap = np.array([-1, 0, 1, -1], dtype=np.int32)
    m, counts = oracle.permute_batched(ids, E=4, E_l=2, max_tokens=3, expert_map=emap)
    assert np.array_equal(m, np.array([[-1, 0], [3, -1], [-1, -1]], dtype=np.int32))
    assert counts.tolist() == [1, 1]
