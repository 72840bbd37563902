"""Pins of the oracle's SLA (v1) options against facts fixed outside it.

The options are the ELU+1 feature map of the linear branch and the output
fusion O = O_s + Proj(O_l) with a learned d x d map (SLA paper summary,
section 4, step 4 and the final-output formula; Eq. 3's symbol list and
Table 2 for the feature map). Each check compares the oracle with a library
routine on a case that reduces to it, a closed form, or a property of the
definition; the scalar brute force in test_oracle_bruteforce.py covers the
general case.
"""

import math

import numpy as np
import pytest
import torch

import oracle as orc


def _elu1_torch(x):
    return (torch.nn.functional.elu(torch.from_numpy(np.ascontiguousarray(x))) + 1.0).numpy()


def _sdpa64(q, k, v):
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x))[None, None]
    return torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v))[0, 0].numpy()


def test_elu1_values_and_library_agreement():
    # phi(0) = 1 from both sides, phi(2) = 3, phi(-1) = 1/e, always positive
    x = np.array([0.0, 2.0, -1.0, -30.0, 1e-300, -1e-300, 5.5])
    f = orc.phi_elu1(x)
    assert f[0] == 1.0 and f[1] == 3.0
    assert abs(f[2] - math.exp(-1.0)) < 1e-16
    assert (f > 0).all()
    rng = np.random.default_rng(1)
    y = 3.0 * rng.standard_normal((64, 32))
    # torch forms expm1(x) + 1: equal up to the rounding of that sum
    np.testing.assert_allclose(orc.phi_elu1(y), _elu1_torch(y), rtol=1e-11, atol=1e-16)


@pytest.mark.parametrize("N,d", [(256, 16), (200, 64)])
def test_all_marginal_elu1_is_linear_attention_in_associative_order(N, d):
    # kh = kl = 0: O_l = phi(Q)(phi(K)^T V) / phi(Q)(phi(K)^T 1) with phi = elu + 1
    rng = np.random.default_rng(N * 3 + d)
    Q, K, V = (rng.standard_normal((1, 1, N, d)) for _ in range(3))
    r = orc.forward(Q, K, V, None, None, [0.0], 0.0, 0.0, feature="elu1")
    fq, fk = _elu1_torch(Q[0, 0]), _elu1_torch(K[0, 0])
    ref = (fq @ (fk.T @ V[0, 0])) / (fq @ fk.sum(axis=0))[:, None]
    np.testing.assert_allclose(r.O_l[(0, 0)], ref, rtol=1e-12, atol=1e-13)


def test_elu1_linear_branch_equals_blocked_h_z_form():
    # Eq. 3 with phi = elu + 1: per-block h_j, z_j summed over the marginal blocks
    rng = np.random.default_rng(12)
    N, d, Nb = 400, 16, 7
    Q, K, V = (rng.standard_normal((1, 1, N, d)) for _ in range(3))
    r = orc.forward(Q, K, V, None, None, [0.5], 2 / 7, 2 / 7, feature="elu1")
    m = r.mask[0, 0]
    fk = _elu1_torch(K[0, 0])
    h = [fk[64 * j:64 * j + 64].T @ V[0, 0, 64 * j:64 * j + 64] for j in range(Nb)]
    z = [fk[64 * j:64 * j + 64].sum(axis=0) for j in range(Nb)]
    for i in range(Nb):
        Hi = sum(h[j] for j in range(Nb) if m[i, j] == 0)
        Zi = sum(z[j] for j in range(Nb) if m[i, j] == 0)
        fq = _elu1_torch(Q[0, 0, 64 * i:64 * i + 64])
        ref = (fq @ Hi) / (fq @ Zi)[:, None]
        np.testing.assert_allclose(r.O_l[(0, 0)][64 * i:64 * i + 64], ref, rtol=1e-12, atol=1e-13)


def test_identity_projection_adds_the_branches_and_zero_keeps_the_sparse_one():
    rng = np.random.default_rng(13)
    N, d = 320, 16
    Q, K, V = (rng.standard_normal((1, 2, N, d)) for _ in range(3))
    rI = orc.forward(Q, K, V, None, None, None, 0.2, 0.2, proj_o=np.eye(d))
    r0 = orc.forward(Q, K, V, None, None, None, 0.2, 0.2, proj_o=np.zeros((d, d)))
    for h in range(2):
        np.testing.assert_allclose(rI.O[(0, h)], rI.O_s[(0, h)] + rI.O_l[(0, h)], rtol=1e-14, atol=0)
        np.testing.assert_array_equal(r0.O[(0, h)], r0.O_s[(0, h)])


def test_constant_values_give_one_plus_column_sums():
    # V == 1: both branches output ones, so O = 1 + 1 @ W = 1 + column sums of W
    # (a transposed W would give its row sums instead)
    rng = np.random.default_rng(14)
    N, d = 300, 16
    Q, K = rng.standard_normal((1, 1, N, d)), rng.standard_normal((1, 1, N, d))
    V = np.ones((1, 1, N, d))
    W = rng.standard_normal((d, d))
    assert abs(W.sum(axis=0) - W.sum(axis=1)).max() > 0.1
    for feature in ("softmax", "elu1"):
        r = orc.forward(Q, K, V, None, None, None, 0.2, 0.2, feature=feature, proj_o=W)
        np.testing.assert_allclose(r.O[(0, 0)], np.broadcast_to(1.0 + W.sum(axis=0), (N, d)),
                                   rtol=1e-12, atol=1e-12)


def test_all_critical_ignores_the_projection():
    # kh = 100%: no marginal block, O_l = 0, so O is dense softmax attention for any W
    rng = np.random.default_rng(15)
    N, d = 256, 16
    Q, K, V = (rng.standard_normal((1, 1, N, d)) for _ in range(3))
    r = orc.forward(Q, K, V, None, None, None, 1.0, 0.0, proj_o=rng.standard_normal((d, d)))
    np.testing.assert_allclose(r.O[(0, 0)], _sdpa64(Q[0, 0], K[0, 0], V[0, 0]), rtol=1e-12, atol=1e-13)


def test_output_is_affine_in_the_projection():
    rng = np.random.default_rng(16)
    N, d = 256, 16
    Q, K, V = (rng.standard_normal((1, 1, N, d)) for _ in range(3))
    W1, W2 = rng.standard_normal((d, d)), rng.standard_normal((d, d))
    f = lambda W: orc.forward(Q, K, V, None, None, None, 0.25, 0.25, feature="elu1", proj_o=W)
    r1, r2, r12 = f(W1), f(W2), f(W1 + 2.0 * W2)
    np.testing.assert_allclose(r12.O[(0, 0)], r1.O[(0, 0)] + 2.0 * (r2.O[(0, 0)] - r2.O_s[(0, 0)]),
                               rtol=1e-11, atol=1e-12)


def test_per_head_projection_uses_each_heads_matrix():
    rng = np.random.default_rng(17)
    N, d, H = 192, 16, 3
    Q, K, V = (rng.standard_normal((1, H, N, d)) for _ in range(3))
    W = rng.standard_normal((H, d, d))
    r = orc.forward(Q, K, V, None, None, None, 0.34, 0.34, proj_o=W)
    for h in range(H):
        rh = orc.forward(Q, K, V, None, None, None, 0.34, 0.34, proj_o=W[h])
        np.testing.assert_array_equal(r.O[(0, h)], rh.O[(0, h)])


def test_no_router_is_the_identity_router():
    rng = np.random.default_rng(18)
    N, d = 330, 16
    Q, K, V = (rng.standard_normal((2, 2, N, d)) for _ in range(3))
    a = orc.forward(Q, K, V, None, None, [0.4, 0.6], 0.2, 0.2)
    b = orc.forward(Q, K, V, np.eye(d), np.eye(d), [0.4, 0.6], 0.2, 0.2)
    np.testing.assert_array_equal(a.mask, b.mask)
    np.testing.assert_array_equal(a.logits, b.logits)
    with pytest.raises(ValueError):
        orc.forward(Q, K, V, np.eye(d), None, [0.4, 0.6], 0.2, 0.2)


def test_elu1_key_offset_changes_the_linear_branch():
    # unlike the softmax map, elu + 1 is not shift-invariant: the softmax map
    # used in its place would make this offset vanish
    rng = np.random.default_rng(19)
    N, d = 256, 16
    Q, K, V = (rng.standard_normal((1, 1, N, d)) for _ in range(3))
    r0 = orc.forward(Q, K, V, None, None, [0.0], 0.0, 0.0, feature="elu1")
    r1 = orc.forward(Q, K + 1.5, V, None, None, [0.0], 0.0, 0.0, feature="elu1")
    assert np.abs(r1.O_l[(0, 0)] - r0.O_l[(0, 0)]).max() > 1e-3
