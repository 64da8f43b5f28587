"""Pins for the oracle's router (softmax -> top-k -> renormalise).

Ties go to the lower expert index; slot order is selection order; the
shared expert of the 513/11 convention is appended with weight 1.0. The
weights are defined with a stated double-precision exp (so that the GPU can
match them bit for bit); these tests hold that exp to exact decimal
arithmetic and the weights to the correctly rounded exact softmax values.
"""
import math
import struct
from decimal import Decimal, getcontext

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


# ---------------------------------------------------------------- exactness

def _ulp(x: float) -> float:
    return math.ulp(x)


def test_route_exp_against_exact_decimal(orc):
    """The stated exp is within 2 ulp of exp(d) computed exactly (60 digits)
    over the whole range the router uses; 0 and the cut-off behave."""
    getcontext().prec = 60
    rng = np.random.default_rng(11)
    ds = np.concatenate([-rng.exponential(3.0, 3000), -rng.uniform(0, 708, 1000),
                         [-0.0, 0.0, -1e-300, -1e-17, -0.5 * math.log(2), -math.log(2), -700.0, -708.0]])
    worst = 0.0
    for d in ds:
        d = float(d)
        got = orc.route_exp(d)
        exact = Decimal(d).exp()
        err = abs(Decimal(got) - exact) / Decimal(_ulp(float(exact)))
        worst = max(worst, float(err))
    assert worst <= 2.0, worst
    assert orc.route_exp(0.0) == 1.0
    assert orc.route_exp(-708.5) == 0.0 and orc.route_exp(-math.inf) == 0.0


def _round_f32_exact(q: Decimal) -> tuple[float, bool]:
    """Nearest fp32 to a positive exact value (ties to even), and whether q
    lies so close to a rounding boundary that 60 digits could not tell."""
    f = float(q)
    f32 = struct.unpack("f", struct.pack("f", f))[0]
    # the two fp32 neighbours bracketing q, then the nearer one
    cands = sorted({f32, float(np.nextafter(np.float32(f32), np.float32(0))),
                    float(np.nextafter(np.float32(f32), np.float32(np.inf)))})
    best = min(cands, key=lambda c: (abs(Decimal(c) - q), int(np.float32(c).view(np.uint32)) & 1))
    ds = sorted(abs(Decimal(c) - q) for c in cands)
    near_tie = ds[1] - ds[0] < q * Decimal(10) ** -40
    return best, near_tie


@pytest.mark.parametrize("renorm", [True, False])
def test_weights_are_correctly_rounded_exact_softmax(orc, renorm):
    """w_j = fp32 nearest to exp(l_j - m) / sum, with the exact exponential
    (60-digit decimal), over 2000 weights from N(0,1) and N(0,4) logits: the
    stated double-precision evaluation rounds to the same fp32 every time."""
    getcontext().prec = 60
    rng = np.random.default_rng(12 + renorm)
    T, E, k = 100, 32, 10
    logits = (rng.standard_normal((T, E)) * rng.choice([1.0, 4.0], (T, 1))).astype(np.float32)
    ids, w = orc.route(logits, k, renorm=renorm)
    mism = 0
    for t in range(T):
        m = Decimal(float(logits[t, ids[t, 0]]))
        ex = [(Decimal(float(v)) - m).exp() for v in logits[t]]
        S = sum(ex[e] for e in ids[t]) if renorm else sum(ex)
        for j in range(k):
            want, near = _round_f32_exact(ex[ids[t, j]] / S)
            assert not near
            mism += float(w[t, j]) != want
    assert mism == 0, f"{mism} weights differ from the correctly rounded exact value"


def test_selection_equals_full_softmax_ranking(orc):
    """Picking the k largest logits equals picking the k largest fp64 softmax
    probabilities (the literal order of the tiny workload's recipe) on
    continuous random logits."""
    rng = np.random.default_rng(13)
    logits = rng.standard_normal((200, 128)).astype(np.float32)
    ids, _ = orc.route(logits, 8)
    p = np.exp(logits.astype(np.float64) - logits.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    order = np.argsort(-p, axis=1, kind="stable")[:, :8]
    assert (order == ids).all()
