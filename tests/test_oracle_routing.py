"""Pins for the oracle's router logits, top-K selection, gate weights and grouping by expert."""
import numpy as np
import pytest
import scipy.special
import torch

from oracle import oracle as O
from tests import _np_ref as R
from workload import SHAPES, make_inputs


def test_logits_match_float64_matmul():
    s = SHAPES["tiny"]
    inp = make_inputs(s, ["x", "w_router"])
    bias = np.linspace(-1, 1, s.E).astype(np.float32)
    got = O.logits(inp["x"], inp["w_router"], bias)
    x = torch.from_numpy(inp["x"].view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    w = torch.from_numpy(inp["w_router"].view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    ref = x @ w.T + bias.astype(np.float64)
    assert np.allclose(got, ref, rtol=0, atol=1e-12)


def _with_ties(rng, T, E):
    lg = rng.standard_normal((T, E)).round(1)      # coarse values: many exact ties
    lg[0, :] = 0.25                                # an all-equal row
    return lg


@pytest.mark.parametrize("T,E,K", [(40, 8, 2), (30, 64, 16), (12, 16, 16), (9, 896, 16), (5, 33, 1)])
def test_select_matches_lexsort(T, E, K):
    lg = _with_ties(np.random.default_rng(E * 100 + K), T, E)
    assert np.array_equal(O.select(lg, K), R.topk_lexsort(lg, K))


def test_select_all_equal_and_k_equals_e():
    lg = np.zeros((2, 10))
    assert np.array_equal(O.select(lg, 10), np.tile(np.arange(10, dtype=np.int32), (2, 1)))
    lg = np.array([[3.0, 1.0, 3.0, 2.0, 3.0]])
    assert O.select(lg, 2).tolist() == [[0, 2]]    # tie at the top: lower indices first
    assert O.select(lg, 4).tolist() == [[0, 2, 4, 3]]


def test_select_rank16_17_tie_goes_to_lower_index():
    rng = np.random.default_rng(5)
    lg = rng.standard_normal((1, 896))
    order = R.topk_lexsort(lg, 17)[0]
    e16, e17 = int(order[15]), int(order[16])
    lg[0, e17] = lg[0, e16]
    ids = O.select(lg, 16)[0]
    assert min(e16, e17) in ids and max(e16, e17) not in ids


def test_route_weights_sum_and_closed_form():
    rng = np.random.default_rng(6)
    lg = rng.standard_normal((50, 64)) * 3
    ids = O.select(lg, 16)
    w = O.route_weights(lg, ids)
    assert np.allclose(w.sum(1), 1.0, atol=1e-12, rtol=0)
    s = scipy.special.expit(np.take_along_axis(lg, ids.astype(np.int64), 1))
    assert np.allclose(w, s / s.sum(1, keepdims=True), rtol=1e-13, atol=0)
    assert np.all(np.diff(w, axis=1) <= 0)         # slots are in rank order
    w1 = O.route_weights(lg, O.select(lg, 1))
    assert np.all(w1 == 1.0)


@pytest.mark.parametrize("T,K,E", [(1, 2, 8), (64, 2, 8), (200, 16, 896), (0, 4, 8)])
def test_permute_matches_library(T, K, E):
    rng = np.random.default_rng(T + K)
    ids = np.stack([rng.choice(E // 2 if E > 8 else E, K, replace=False) for _ in range(T)]) \
        if T else np.zeros((0, K), np.int64)
    ids = ids.astype(np.int32).reshape(T, K)
    p = O.permute(ids, E)
    flat = ids.reshape(-1)
    assert np.array_equal(p.counts, np.bincount(flat, minlength=E))
    assert p.offsets[0] == 0 and p.offsets[-1] == T * K
    assert np.array_equal(np.diff(p.offsets), p.counts)
    assert np.array_equal(p.sorted_pairs, np.argsort(flat, kind="stable"))
    assert np.array_equal(p.inv[p.sorted_pairs], np.arange(T * K))
    if E > 8 and T:
        assert np.sum(p.counts == 0) >= E // 2     # experts with no pairs keep empty ranges
