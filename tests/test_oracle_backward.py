"""Pins of the backward oracle (oracle/backward.py): the torch re-statement of
the forward against the pinned numpy oracle, autograd against central finite
differences, the mixing ratio's gradient against its closed form, and the
all-critical case against the autograd of torch's own attention routine."""

import numpy as np
import pytest
import torch

import oracle as orc
from oracle import backward as ob


def _case(N, d, H=2, seed=0):
    rng = np.random.default_rng(seed)
    Q, K, V = (rng.standard_normal((1, H, N, d)) for _ in range(3))
    Nb = (N + 63) // 64
    mask = rng.choice(np.array([1, 0, -1], dtype=np.int8), size=(1, H, Nb, Nb))
    mask[..., 0] = 1            # every row has a critical block
    mask[..., Nb - 1] = 0       # and a marginal one (the ragged block when N % 64)
    alpha = rng.uniform(0.2, 0.8, size=H)
    dO = rng.standard_normal((1, H, N, d))
    return Q, K, V, alpha, mask, dO


@pytest.mark.parametrize("phi", ["softmax", "elu1"])
def test_torch_forward_equals_the_numpy_oracle(phi):
    Q, K, V, alpha, mask, _ = _case(200, 16)
    t = lambda x: torch.from_numpy(x)
    O, Os, Ol = ob.forward_torch(t(Q), t(K), t(V), t(alpha), mask, phi)
    r = orc.forward(Q, K, V, np.eye(16), np.eye(16), alpha, 0.0, 0.0, mask_in=mask, feature=phi)
    for h in range(2):
        np.testing.assert_allclose(O[0, h].numpy(), r.O[(0, h)], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(Os[0, h].numpy(), r.O_s[(0, h)], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(Ol[0, h].numpy(), r.O_l[(0, h)], rtol=1e-12, atol=1e-13)


def test_gradients_against_finite_differences():
    Q, K, V, alpha, mask, dO = _case(70, 8, H=1, seed=3)
    g = ob.backward(Q, K, V, alpha, mask, dO)
    t = lambda x: torch.from_numpy(np.array(x))

    def loss(Q_, K_, V_, a_):
        O, _, _ = ob.forward_torch(t(Q_), t(K_), t(V_), t(a_), mask)
        return float((O.numpy() * dO).sum())

    rng = np.random.default_rng(4)
    eps = 1e-6
    for name, arr, idx in [("dQ", Q, 0), ("dK", K, 1), ("dV", V, 2)]:
        for _ in range(6):
            pos = tuple(int(rng.integers(0, s)) for s in arr.shape)
            args = [Q, K, V, alpha]
            plus = [a.copy() for a in args]
            minus = [a.copy() for a in args]
            plus[idx][pos] += eps
            minus[idx][pos] -= eps
            fd = (loss(*plus) - loss(*minus)) / (2 * eps)
            assert abs(fd - g[name][pos]) <= 1e-6 * max(1.0, abs(fd)), (name, pos, fd, g[name][pos])
    ap, am = alpha.copy(), alpha.copy()
    ap[0] += eps
    am[0] -= eps
    fd = (loss(Q, K, V, ap) - loss(Q, K, V, am)) / (2 * eps)
    assert abs(fd - g["dalpha"][0]) <= 1e-6 * max(1.0, abs(fd))


def test_alpha_gradient_closed_form():
    # O = alpha O_s + (1 - alpha) O_l: dL/dalpha_h = sum dO * (O_s - O_l) over the head
    Q, K, V, alpha, mask, dO = _case(260, 16, H=3, seed=5)
    g = ob.backward(Q, K, V, alpha, mask, dO)
    r = orc.forward(Q, K, V, np.eye(16), np.eye(16), alpha, 0.0, 0.0, mask_in=mask)
    for h in range(3):
        ref = float((dO[0, h] * (r.O_s[(0, h)] - r.O_l[(0, h)])).sum())
        assert abs(g["dalpha"][h] - ref) <= 1e-10 * max(1.0, abs(ref))


def test_all_critical_equals_attention_autograd():
    # every block critical, alpha = 1: the gradients of dense softmax attention
    rng = np.random.default_rng(6)
    N, d = 192, 16
    Q, K, V, dO = (rng.standard_normal((1, 1, N, d)) for _ in range(4))
    mask = np.ones((1, 1, 3, 3), dtype=np.int8)
    g = ob.backward(Q, K, V, np.ones(1), mask, dO)
    q, k, v = (torch.from_numpy(x).requires_grad_(True) for x in (Q, K, V))
    out = torch.nn.functional.scaled_dot_product_attention(q, k, v)
    (out * torch.from_numpy(dO)).sum().backward()
    for name, t in (("dQ", q), ("dK", k), ("dV", v)):
        np.testing.assert_allclose(g[name], t.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_dq_rows_equal_the_full_gradient():
    Q, K, V, alpha, mask, dO = _case(300, 16, H=2, seed=9)
    g = ob.backward(Q, K, V, alpha, mask, dO)
    rows = ob.dq_rows(Q, K, V, alpha, mask, dO, 0, 1, [0, 2, 4])
    for i, r in rows.items():
        np.testing.assert_allclose(r, g["dQ"][0, 1, 64 * i:64 * i + 64], rtol=1e-11, atol=1e-13)


def test_value_gradient_sum_closed_form():
    # both branches are row-normalised maps of V: summed over the keys, dV is
    # sum_t (alpha [t has a critical block] + (1 - alpha) [t has a marginal one]) dO[t]
    Q, K, V, alpha, mask, dO = _case(330, 16, H=2, seed=10)
    mask[0, 1, 2] = -1
    mask[0, 1, 3, :] = 1
    g = ob.backward(Q, K, V, alpha, mask, dO)
    for h in range(2):
        c = np.repeat((mask[0, h] == 1).any(axis=1), 64)[:330].astype(float)
        m = np.repeat((mask[0, h] == 0).any(axis=1), 64)[:330].astype(float)
        w = alpha[h] * c + (1 - alpha[h]) * m
        np.testing.assert_allclose(g["dV"][0, h].sum(axis=0), (w[:, None] * dO[0, h]).sum(axis=0),
                                   rtol=1e-11, atol=1e-11)


# ---- the SLA formulation (O = O_s + O_l W) and the ELU+1 feature map

def _fd_check(Q, K, V, mask, dO, g, phi, proj_o=None, alpha=None, n=5, seed=11):
    t = lambda x: torch.from_numpy(np.array(x))

    def loss(Q_, K_, V_, W_):
        O, _, _ = ob.forward_torch(t(Q_), t(K_), t(V_), None if alpha is None else t(alpha), mask, phi,
                                   None if W_ is None else t(W_))
        return float((O.numpy() * dO).sum())

    rng = np.random.default_rng(seed)
    eps = 1e-6
    args = [Q, K, V, proj_o]
    names = ["dQ", "dK", "dV"] + (["dproj_o"] if proj_o is not None else [])
    for idx, name in enumerate(names):
        arr = args[idx]
        for _ in range(n):
            pos = tuple(int(rng.integers(0, s)) for s in arr.shape)
            plus = [None if a is None else a.copy() for a in args]
            minus = [None if a is None else a.copy() for a in args]
            plus[idx][pos] += eps
            minus[idx][pos] -= eps
            fd = (loss(*plus) - loss(*minus)) / (2 * eps)
            assert abs(fd - g[name][pos]) <= 1e-6 * max(1.0, abs(fd)), (name, pos, fd, g[name][pos])


@pytest.mark.parametrize("phi", ["softmax", "elu1"])
@pytest.mark.parametrize("per_head", [False, True])
def test_sla1_gradients_against_finite_differences(phi, per_head):
    Q, K, V, _, mask, dO = _case(70, 8, H=2, seed=12)
    rng = np.random.default_rng(13)
    W = rng.standard_normal((2, 8, 8) if per_head else (8, 8)) / np.sqrt(8)
    g = ob.backward(Q, K, V, None, mask, dO, phi=phi, proj_o=W)
    assert g["dproj_o"].shape == W.shape and "dalpha" not in g
    _fd_check(Q, K, V, mask, dO, g, phi, proj_o=W)


def test_elu1_gradients_against_finite_differences():
    Q, K, V, alpha, mask, dO = _case(70, 8, H=1, seed=14)
    g = ob.backward(Q, K, V, alpha, mask, dO, phi="elu1")
    _fd_check(Q, K, V, mask, dO, g, "elu1", alpha=alpha)


@pytest.mark.parametrize("phi", ["softmax", "elu1"])
def test_sla1_identity_map_is_twice_the_half_mix(phi):
    # W = I gives O = O_s + O_l = 2 (0.5 O_s + 0.5 O_l): every input gradient doubles
    Q, K, V, _, mask, dO = _case(150, 16, H=2, seed=15)
    g1 = ob.backward(Q, K, V, None, mask, dO, phi=phi, proj_o=np.eye(16))
    g2 = ob.backward(Q, K, V, np.full(2, 0.5), mask, dO, phi=phi)
    for name in ("dQ", "dK", "dV"):
        np.testing.assert_allclose(g1[name], 2.0 * g2[name], rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("per_head", [False, True])
def test_sla1_map_gradient_closed_form(per_head):
    # O is linear in W: dL/dW = sum over tokens (and batches, and heads when W is shared) of O_l^T dO
    Q, K, V, _, mask, dO = _case(200, 16, H=3, seed=16)
    W = np.random.default_rng(17).standard_normal((3, 16, 16) if per_head else (16, 16))
    g = ob.backward(Q, K, V, None, mask, dO, proj_o=W)
    r = orc.forward(Q, K, V, None, None, None, 0.0, 0.0, mask_in=mask, proj_o=W)
    per = np.stack([r.O_l[(0, h)].T @ dO[0, h] for h in range(3)])
    np.testing.assert_allclose(g["dproj_o"], per if per_head else per.sum(axis=0), rtol=1e-10, atol=1e-11)


def test_sla1_dq_rows_equal_the_full_gradient():
    Q, K, V, _, mask, dO = _case(300, 16, H=2, seed=18)
    W = np.random.default_rng(19).standard_normal((16, 16))
    g = ob.backward(Q, K, V, None, mask, dO, phi="elu1", proj_o=W)
    rows = ob.dq_rows(Q, K, V, None, mask, dO, 0, 1, [0, 3, 4], phi="elu1", proj_o=W)
    for i, r in rows.items():
        np.testing.assert_allclose(r, g["dQ"][0, 1, 64 * i:64 * i + 64], rtol=1e-11, atol=1e-13)
