"""Pins of the oracle's SoftTop-k (SLA2 article, the two-stage training
paragraphs, stage 1; SLA2 cross-paper synthesis, §3 on the binary search for
lambda_i): M[i, j] = sigmoid((Pc[i, j] - lambda_i) / tau) with every row
summing to k. Each check is a property the definition fixes, a limit with a
closed form, or an independent library root finder."""

import numpy as np
import pytest
import scipy.optimize
import scipy.special

import oracle as orc


def _rows(shape, seed, scale=3.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


@pytest.mark.parametrize("k", [1, 2.5, 7, 49])
@pytest.mark.parametrize("tau", [1e-4, 1e-2, 1.0])
def test_rows_sum_to_k(k, tau):
    M, lam = orc.soft_topk(_rows((4, 50), 1), k, tau)
    np.testing.assert_allclose(M.sum(axis=-1), k, rtol=1e-12, atol=1e-12)
    assert ((M >= 0) & (M <= 1)).all() and np.isfinite(lam).all()  # saturates at small tau


def test_lambda_against_a_library_root_finder():
    s = _rows((6, 40), 2)
    P = np.exp(s - s.max(-1, keepdims=True))
    P /= P.sum(-1, keepdims=True)
    k, tau = 4.0, 3e-3
    _, lam = orc.soft_topk(s, k, tau)
    for i in range(6):
        f = lambda x: scipy.special.expit((P[i] - x) / tau).sum() - k
        ref = scipy.optimize.brentq(f, P[i].min() - 1.0, P[i].max() + 1.0, xtol=1e-15, rtol=1e-15)
        assert abs(lam[i] - ref) <= 1e-12 * max(1.0, abs(ref)) + 1e-15


def test_small_temperature_is_the_hard_top_k():
    # a gap between the k-th and (k+1)-th largest Pc: as tau -> 0 the weights
    # become the critical set of Eq. 2 (ties broken by index do not arise)
    s = _rows((5, 64), 3)
    n_h = 6
    hard = orc.classify(s, n_h, 0) == 1
    M, _ = orc.soft_topk(s, n_h, 1e-9)
    np.testing.assert_allclose(M, hard.astype(float), atol=1e-6)


def test_large_temperature_is_uniform():
    s = _rows((3, 32), 4)
    M, _ = orc.soft_topk(s, 5, 1e6)
    np.testing.assert_allclose(M, 5 / 32, rtol=1e-6)


def test_weights_follow_the_row_order():
    s = _rows((4, 60), 5)
    M, _ = orc.soft_topk(s, 8, 1e-3)
    for i in range(4):
        o = np.argsort(-s[i], kind="stable")
        assert (np.diff(M[i][o]) <= 1e-15).all()


def test_logit_shift_and_temperature_scaling():
    # a constant added to a row's logits leaves Pc and so M unchanged;
    # M(Pc, tau) is a function of (Pc - lambda) / tau only, so lambda moves
    # with tau as the closed form of one uniform row shows
    s = _rows((3, 30), 6)
    a, _ = orc.soft_topk(s, 3, 2e-3)
    b, _ = orc.soft_topk(s + 11.0, 3, 2e-3)
    np.testing.assert_allclose(a, b, atol=1e-12)
    u, lam = orc.soft_topk(np.zeros((1, 10)), 3, 0.5)  # Pc = 0.1 everywhere
    np.testing.assert_allclose(u, 0.3, rtol=1e-12)
    # sigmoid((0.1 - lambda) / 0.5) = 0.3  ->  lambda = 0.1 - 0.5 * logit(0.3)
    assert abs(lam[0] - (0.1 - 0.5 * np.log(0.3 / 0.7))) < 1e-12


def test_edge_budgets():
    s = _rows((2, 16), 7)
    z, lz = orc.soft_topk(s, 0, 1e-2)
    o, lo = orc.soft_topk(s, 16, 1e-2)
    assert (z == 0).all() and np.isposinf(lz).all()
    assert (o == 1).all() and np.isneginf(lo).all()
    with pytest.raises(ValueError):
        orc.soft_topk(s, 17, 1e-2)
    with pytest.raises(ValueError):
        orc.soft_topk(s, 3, 0.0)
