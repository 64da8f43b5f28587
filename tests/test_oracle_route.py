"""Pins for the oracle's router (softmax -> top-k -> renormalise).

Ties go to the lower expert index; slot order is selection order; the
shared expert of the 513/11 convention is appended with weight 1.0.
"""
import math

import numpy as np
import pytest


def _brute_ids(logits_row, k):
    # Independent criterion: rank by logit (softmax is monotone), then index.
    order = sorted(range(len(logits_row)), key=lambda e: (-float(logits_row[e]), e))
    return order[:k]


@pytest.mark.parametrize("T,E,k", [(64, 8, 2), (37, 128, 8), (5, 512, 10)])
def test_ids_match_brute_force(orc, T, E, k):
    rng = np.random.default_rng(T * E + k)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    ids, w = orc.route(logits, k)
    for t in range(T):
        assert list(ids[t]) == _brute_ids(logits[t], k)


def test_weight_ratios_are_exp_of_logit_gaps(orc):
    rng = np.random.default_rng(1)
    logits = rng.standard_normal((50, 16)).astype(np.float32)
    ids, w = orc.route(logits, 4)
    for t in range(50):
        l = [float(logits[t, e]) for e in ids[t]]
        for j in range(1, 4):
            assert w[t, j] / w[t, 0] == pytest.approx(math.exp(l[j] - l[0]), rel=1e-6)
        assert float(np.sum(w[t].astype(np.float64))) == pytest.approx(1.0, abs=4 * 2 ** -24)


def test_equal_logits_give_lowest_ids_and_uniform_weights(orc):
    for k in (1, 2, 4, 8):
        logits = np.full((3, 16), 0.7, dtype=np.float32)
        ids, w = orc.route(logits, k)
        assert (ids == np.arange(k, dtype=np.int32)[None, :]).all()
        assert (w == np.float32(1.0 / k)).all()   # exact for powers of two


def test_dominant_logit_takes_slot_zero(orc):
    rng = np.random.default_rng(2)
    logits = rng.standard_normal((20, 64)).astype(np.float32)
    hot = rng.integers(0, 64, size=20)
    logits[np.arange(20), hot] = 50.0
    ids, w = orc.route(logits, 8)
    assert (ids[:, 0] == hot).all()
    assert (w[:, 0] > 0.999).all()


def test_without_renorm_weights_are_full_softmax(orc):
    rng = np.random.default_rng(3)
    logits = rng.standard_normal((10, 32)).astype(np.float32)
    ids, w = orc.route(logits, 4, renorm=False)
    for t in range(10):
        z = sum(math.exp(float(v)) for v in logits[t])
        for j in range(4):
            assert w[t, j] == pytest.approx(math.exp(float(logits[t, ids[t, j]])) / z, rel=1e-6)


def test_shared_expert_appended(orc):
    rng = np.random.default_rng(4)
    logits = rng.standard_normal((9, 512)).astype(np.float32)
    ids, w = orc.route(logits, 10, shared_id=512, shared_w=1.0)
    assert ids.shape == (9, 11)
    assert (ids[:, 10] == 512).all() and (w[:, 10] == 1.0).all()
    ids10, w10 = orc.route(logits, 10)
    assert (ids[:, :10] == ids10).all() and (w[:, :10] == w10).all()


def test_masked_experts_never_chosen(orc):
    rng = np.random.default_rng(5)
    logits = rng.standard_normal((30, 128)).astype(np.float32)
    logits[:, 124:] = -np.inf
    ids, w = orc.route(logits, 8)
    assert (ids < 124).all() and np.isfinite(w).all()


def test_strided_logits_equal_contiguous(orc):
    rng = np.random.default_rng(6)
    buf = rng.standard_normal((128, 40)).astype(np.float32)
    logits = buf.T                       # [40, 128], strides (4, 160)
    a = orc.route(logits, 8)
    b = orc.route(np.ascontiguousarray(logits), 8)
    assert (a[0] == b[0]).all() and (a[1] == b[1]).all()
