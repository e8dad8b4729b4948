"""Pins of the oracle's router (the [Router] stage of the modular-kernel page;
weights already carrying the routed scaling factor per the output-contract
page).  Ids are pinned by brute force (a full lexicographic sort per token, and
torch.topk on tie-free inputs); weights by closed forms and by torch's own
softmax/sigmoid in float64."""
import numpy as np
import pytest
import torch

import oracle
import synth


def _brute_ids(logits, k):
    T, E = logits.shape
    ids = np.empty((T, k), dtype=np.int32)
    for t in range(T):
        order = np.lexsort((np.arange(E), -logits[t].astype(np.float64)))
        ids[t] = order[:k]
    return ids


@pytest.mark.parametrize("T,E,k", [(16, 8, 2), (33, 256, 8), (5, 8, 8), (7, 3, 1)])
def test_ids_match_full_sort(T, E, k):
    logits = synth.normal_f32(21, 1, (T, E))
    ids, _ = oracle.route(logits, k, oracle.SOFTMAX, True, 1.0)
    assert np.array_equal(ids, _brute_ids(logits, k))


def test_ids_match_torch_topk_when_tie_free():
    logits = synth.normal_f32(22, 1, (64, 256))
    assert all(len(np.unique(r)) == r.size for r in logits)
    ids, _ = oracle.route(logits, 8, oracle.SIGMOID, True, 2.5)
    ref = torch.topk(torch.from_numpy(logits), 8, dim=1, sorted=True).indices.numpy()
    assert np.array_equal(ids, ref)


def test_ties_go_to_the_smaller_expert_id():
    logits = np.array([[1.0, 3.0, 3.0, 0.0],
                       [2.0, 2.0, 2.0, 2.0],
                       [-1.0, 5.0, -1.0, 5.0]], dtype=np.float32)
    ids, w = oracle.route(logits, 2, oracle.SOFTMAX, True, 1.0)
    assert ids.tolist() == [[1, 2], [0, 1], [1, 3]]
    assert np.all(w == 0.5)
    ids, w = oracle.route(logits, 3, oracle.SIGMOID, True, 2.5)
    assert ids.tolist() == [[1, 2, 0], [0, 1, 2], [1, 3, 0]]
    np.testing.assert_allclose(w[1], 2.5 / 3, rtol=1e-15, atol=0)


def test_softmax_renormalized_closed_form():
    logits = synth.normal_f32(23, 1, (50, 8))
    _, w = oracle.route(logits, 2, oracle.SOFTMAX, True, 1.0)
    assert np.allclose(w.sum(1), 1.0, rtol=0, atol=1e-15)
    p = torch.softmax(torch.from_numpy(logits).double(), dim=1).numpy()
    ids = _brute_ids(logits, 2)
    sel = np.take_along_axis(p, ids, 1)
    assert np.allclose(w, sel / sel.sum(1, keepdims=True), rtol=1e-14, atol=0)


def test_softmax_all_experts_equals_softmax():
    logits = synth.normal_f32(24, 1, (20, 8))
    ids, w = oracle.route(logits, 8, oracle.SOFTMAX, False, 1.0)
    p = torch.softmax(torch.from_numpy(logits).double(), dim=1).numpy()
    assert np.allclose(w, np.take_along_axis(p, ids, 1), rtol=1e-14, atol=0)
    # k = E with renormalization changes nothing
    _, w2 = oracle.route(logits, 8, oracle.SOFTMAX, True, 1.0)
    assert np.allclose(w, w2, rtol=1e-14, atol=0)


def test_sigmoid_renormalized_scaled_closed_form():
    logits = synth.normal_f32(25, 1, (40, 256))
    ids, w = oracle.route(logits, 8, oracle.SIGMOID, True, 2.5)
    assert np.allclose(w.sum(1), 2.5, rtol=0, atol=1e-14)
    s = torch.sigmoid(torch.from_numpy(logits).double()).numpy()
    sel = np.take_along_axis(s, ids, 1)
    assert np.allclose(w, 2.5 * sel / sel.sum(1, keepdims=True), rtol=1e-14, atol=0)
    # without renormalization: the raw scores times rsf
    _, w_raw = oracle.route(logits, 8, oracle.SIGMOID, False, 2.5)
    assert np.allclose(w_raw, 2.5 * sel, rtol=1e-14, atol=0)


def test_top1_weight_is_exactly_one():
    logits = synth.normal_f32(26, 1, (10, 8))
    _, w = oracle.route(logits, 1, oracle.SOFTMAX, True, 1.0)
    assert np.all(w == 1.0)
