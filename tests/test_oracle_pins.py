"""Pins of the float64 oracle against facts fixed outside it.

Every check here compares the oracle with something it does not compute itself:
closed forms, a library routine on a special case that reduces to it, an
invariance of the method, or an independent scalar brute force (in
test_oracle_bruteforce.py).
"""

import math

import numpy as np
import pytest
import torch

import oracle as orc

RNG = np.random.default_rng(12345)


def _rand(*shape, rng=RNG):
    return rng.standard_normal(shape)


# ----------------------------------------------------------------- block counts

@pytest.mark.parametrize("Nb", [1, 2, 7, 16, 100, 128, 512, 1182])
@pytest.mark.parametrize("kh,kl", [(0.05, 0.10), (0.03, 0.10), (0.25, 0.25), (0.0, 0.0),
                                   (1.0, 0.0), (0.0, 1.0), (0.5, 0.5), (0.29, 0.0)])
def test_block_counts_floor_property(Nb, kh, kl):
    if kh + kl > 1.0 + 1e-12:
        pytest.skip("inconsistent fractions")
    try:
        n_h, n_l = orc.block_counts(Nb, kh, kl)
    except ValueError:
        # only legitimate when the floors (with the min-1 rule) overflow the row
        assert max(1, math.floor(kh * Nb + 1e-9)) + math.floor(kl * Nb + 1e-9) > Nb
        return
    # n_h is the largest count whose share does not exceed kh (at least 1 if kh > 0)
    if kh > 0:
        assert n_h >= 1
        if n_h > 1:
            assert n_h <= kh * Nb + 1e-9 < n_h + 1
    else:
        assert n_h == 0
    assert n_l <= kl * Nb + 1e-9 < n_l + 1
    assert n_h + n_l <= Nb


def test_block_counts_examples_from_configs():
    # the workloads' realised sparsities 1 - n_h/Nb reach at least the nominal one
    assert orc.block_counts(16, 0.25, 0.25) == (4, 4)
    assert orc.block_counts(100, 0.29, 0.0)[0] == 29  # 0.29*100 = 28.999... in binary
    for Nb, kh in ((128, 0.05), (512, 0.05), (512, 0.03), (1182, 0.03)):
        n_h, _ = orc.block_counts(Nb, kh, 0.10)
        assert 1 - n_h / Nb >= 1 - kh


def test_block_counts_rejects_overflow_and_range():
    with pytest.raises(ValueError):
        orc.block_counts(10, 0.6, 0.5)
    with pytest.raises(ValueError):
        orc.block_counts(10, -0.1, 0.0)
    with pytest.raises(ValueError):
        orc.block_counts(10, 0.1, 1.5)


# ------------------------------------------------------------- router + pooling

@pytest.mark.parametrize("N", [64, 100, 200, 256])
def test_pool_of_constant_blocks_is_the_constant(N):
    d = 8
    Nb = orc.num_blocks(N)
    consts = _rand(Nb, d)
    X = np.repeat(consts, 64, axis=0)[:N]
    np.testing.assert_allclose(orc.router_pool(X, np.eye(d)), consts, rtol=0, atol=1e-14)


@pytest.mark.parametrize("N", [64, 100, 130])
def test_pool_of_a_ramp_is_the_block_midpoint(N):
    # X[t] = t * u: the mean over tokens [a, b) is (a + b - 1)/2 * u, also for a ragged tail
    d = 4
    u = np.array([1.0, -2.0, 0.5, 3.0])
    X = np.arange(N, dtype=np.float64)[:, None] * u[None, :]
    pooled = orc.router_pool(X, np.eye(d))
    for i in range(orc.num_blocks(N)):
        a, b = 64 * i, min(64 * i + 64, N)
        np.testing.assert_allclose(pooled[i], (a + b - 1) / 2.0 * u, rtol=1e-15, atol=0)


def test_router_orientation_in_out():
    # proj[in, out]: a matrix moving input feature 0 to output feature 2 only
    d = 4
    P = np.zeros((d, d))
    P[0, 2] = 3.0
    X = _rand(64, d)
    pooled = orc.router_pool(X, P)
    np.testing.assert_allclose(pooled[0], [0.0, 0.0, 3.0 * X[:, 0].mean(), 0.0], atol=1e-15)


def test_pool_then_project_equals_project_then_pool():
    d = 16
    X = _rand(200, d)
    P = _rand(d, d)
    np.testing.assert_allclose(orc.router_pool(X, P), orc.router_pool(X, np.eye(d)) @ P,
                               rtol=1e-12, atol=1e-13)


# ------------------------------------------------------------ compressed scores

def test_pc_rows_sum_to_one_and_logit_closed_form():
    d = 16
    qbar = _rand(5, d)
    kbar = _rand(7, d)
    s, Pc = orc.compressed_scores(qbar, kbar, d)
    np.testing.assert_allclose(Pc.sum(axis=1), 1.0, atol=1e-15)
    # one entry written as an explicit scalar sum
    ref = sum(qbar[2, c] * kbar[4, c] for c in range(d)) / 4.0
    assert abs(s[2, 4] - ref) < 1e-13


def test_pc_shift_invariance():
    # adding c*w to every pooled key (w fixed) shifts each logit row by a constant
    d = 8
    qbar, kbar = _rand(4, d), _rand(9, d)
    w = _rand(d)
    _, Pc0 = orc.compressed_scores(qbar, kbar, d)
    _, Pc1 = orc.compressed_scores(qbar, kbar + 2.5 * w[None, :], d)
    np.testing.assert_allclose(Pc0, Pc1, rtol=1e-12, atol=1e-15)


# --------------------------------------------------------------- classification

def _brute_rank_mask(s, n_h, n_l):
    import functools
    Nq, Nk = s.shape
    out = np.zeros((Nq, Nk), dtype=np.int8)
    for i in range(Nq):
        def cmp(a, b):
            if s[i, a] != s[i, b]:
                return -1 if s[i, a] > s[i, b] else 1
            return -1 if a < b else (1 if a > b else 0)
        order = sorted(range(Nk), key=functools.cmp_to_key(cmp))
        for r, j in enumerate(order):
            out[i, j] = 1 if r < n_h else (-1 if r >= Nk - n_l else 0)
    return out


@pytest.mark.parametrize("Nk,n_h,n_l", [(16, 4, 4), (9, 1, 3), (12, 0, 5), (12, 12, 0), (10, 3, 7)])
def test_classify_matches_comparator_sort_with_ties(Nk, n_h, n_l):
    rng = np.random.default_rng(Nk * 100 + n_h)
    s = np.round(rng.standard_normal((6, Nk)), 1)  # few distinct values: many exact ties
    np.testing.assert_array_equal(orc.classify(s, n_h, n_l), _brute_rank_mask(s, n_h, n_l))


def test_classify_counts_per_row():
    s = _rand(20, 37)
    m = orc.classify(s, 5, 11)
    assert ((m == 1).sum(axis=1) == 5).all()
    assert ((m == -1).sum(axis=1) == 11).all()
    # critical entries hold the largest logits, negligible the smallest
    for i in range(20):
        assert s[i][m[i] == 1].min() > s[i][m[i] == 0].max() > s[i][m[i] == -1].max()


def test_zero_queries_give_index_order_mask():
    # Q == 0: every logit is 0, the order is the block index
    B, H, N, d = 1, 1, 64 * 10, 8
    Q = np.zeros((B, H, N, d))
    K = _rand(B, H, N, d)
    V = _rand(B, H, N, d)
    r = orc.forward(Q, K, V, np.eye(d), np.eye(d), [0.5], 0.3, 0.2, compute_outputs=False)
    expect = np.array([1] * 3 + [0] * 5 + [-1] * 2, dtype=np.int8)
    for i in range(10):
        np.testing.assert_array_equal(r.mask[0, 0, i], expect)


def test_key_block_permutation_permutes_mask_columns():
    B, H, Nb, d = 1, 1, 8, 8
    N = 64 * Nb
    Q, K, V = _rand(B, H, N, d), _rand(B, H, N, d), _rand(B, H, N, d)
    perm = np.random.default_rng(7).permutation(Nb)
    Kp = K.reshape(B, H, Nb, 64, d)[:, :, perm].reshape(B, H, N, d)
    r0 = orc.forward(Q, K, V, np.eye(d), np.eye(d), [0.5], 0.25, 0.25, compute_outputs=False)
    r1 = orc.forward(Q, Kp, V, np.eye(d), np.eye(d), [0.5], 0.25, 0.25, compute_outputs=False)
    np.testing.assert_array_equal(r1.mask[0, 0], r0.mask[0, 0][:, perm])


# --------------------------------------------------------------- sparse branch

def _sdpa64(q, k, v, attn_mask=None):
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x))[None, None]
    m = None if attn_mask is None else torch.from_numpy(attn_mask)
    out = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=m)
    return out[0, 0].numpy()


@pytest.mark.parametrize("N,d", [(256, 16), (300, 32)])
def test_all_critical_is_dense_softmax_attention(N, d):
    # kh = 100%: every block critical, O_s is dense softmax attention (Full Attention)
    rng = np.random.default_rng(N)
    Q, K, V = (rng.standard_normal((1, 1, N, d)) for _ in range(3))
    r = orc.forward(Q, K, V, np.eye(d), np.eye(d), [1.0], 1.0, 0.0)
    ref = _sdpa64(Q[0, 0], K[0, 0], V[0, 0])
    np.testing.assert_allclose(r.O_s[(0, 0)], ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(r.O[(0, 0)], ref, rtol=1e-12, atol=1e-13)  # alpha = 1


def test_sparse_branch_equals_sdpa_with_expanded_token_mask():
    rng = np.random.default_rng(3)
    N, d, Nb = 320, 16, 5
    Q, K, V = (rng.standard_normal((1, 1, N, d)) for _ in range(3))
    mask = rng.choice([1, 0, -1], size=(1, 1, Nb, Nb)).astype(np.int8)
    mask[0, 0, :, 0] = 1  # every row keeps one critical block
    r = orc.forward(Q, K, V, np.eye(d), np.eye(d), [1.0], 0.2, 0.2, mask_in=mask)
    tok = np.repeat(np.repeat(mask[0, 0] == 1, 64, axis=0), 64, axis=1)[:N, :N]
    ref = _sdpa64(Q[0, 0], K[0, 0], V[0, 0], attn_mask=tok)
    np.testing.assert_allclose(r.O_s[(0, 0)], ref, rtol=1e-12, atol=1e-13)


# --------------------------------------------------------------- linear branch

def _phi(x):
    e = np.exp(x - x.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


@pytest.mark.parametrize("N,d", [(256, 16), (200, 64)])
def test_all_marginal_is_linear_attention_in_associative_order(N, d):
    # kh = kl = 0: every block marginal, O_l = phi(Q)(phi(K)^T V) / phi(Q)(phi(K)^T 1)
    rng = np.random.default_rng(N + d)
    Q, K, V = (rng.standard_normal((1, 1, N, d)) for _ in range(3))
    r = orc.forward(Q, K, V, np.eye(d), np.eye(d), [0.0], 0.0, 0.0)
    fq, fk = _phi(Q[0, 0]), _phi(K[0, 0])
    ref = (fq @ (fk.T @ V[0, 0])) / (fq @ fk.sum(axis=0))[:, None]
    np.testing.assert_allclose(r.O_l[(0, 0)], ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(r.O[(0, 0)], ref, rtol=1e-12, atol=1e-13)  # alpha = 0
    assert not r.O_s[(0, 0)].any()  # no critical block: zero sparse output


def test_linear_branch_equals_blocked_h_z_form():
    # Eq. 3: H_i = sum over marginal j of phi(K_j)^T V_j, Z_i likewise, O_l = phi(Q_i)H_i / phi(Q_i)Z_i
    rng = np.random.default_rng(11)
    N, d = 448, 16
    Nb = 7
    Q, K, V = (rng.standard_normal((1, 1, N, d)) for _ in range(3))
    r = orc.forward(Q, K, V, np.eye(d), np.eye(d), [0.3], 2 / 7, 1 / 7)
    m = r.mask[0, 0]
    fk = _phi(K[0, 0])
    h = [fk[64 * j:64 * j + 64].T @ V[0, 0, 64 * j:64 * j + 64] for j in range(Nb)]
    z = [fk[64 * j:64 * j + 64].sum(axis=0) for j in range(Nb)]
    Htot, Ztot = sum(h), sum(z)
    for i in range(Nb):
        Hi = sum(h[j] for j in range(Nb) if m[i, j] == 0)
        Zi = sum(z[j] for j in range(Nb) if m[i, j] == 0)
        # "total minus excluded" gives the same sums
        Hx = Htot - sum((h[j] for j in range(Nb) if m[i, j] != 0), np.zeros((d, d)))
        np.testing.assert_allclose(Hx, Hi, rtol=1e-12, atol=1e-12)
        fq = _phi(Q[0, 0, 64 * i:64 * i + 64])
        ref = (fq @ Hi) / (fq @ Zi)[:, None]
        np.testing.assert_allclose(r.O_l[(0, 0)][64 * i:64 * i + 64], ref, rtol=1e-12, atol=1e-13)
        assert abs((Ztot - sum((z[j] for j in range(Nb) if m[i, j] != 0), np.zeros(d)) - Zi).max()) < 1e-12


# ------------------------------------------------------------------------ mix

def test_mix_is_affine_in_alpha():
    rng = np.random.default_rng(5)
    N, d = 256, 16
    Q, K, V = (rng.standard_normal((1, 2, N, d)) for _ in range(3))
    r0 = orc.forward(Q, K, V, np.eye(d), np.eye(d), [0.0, 1.0], 0.25, 0.25)
    r1 = orc.forward(Q, K, V, np.eye(d), np.eye(d), [0.7, 0.2], 0.25, 0.25)
    for h, a in ((0, 0.7), (1, 0.2)):
        Os, Ol = r0.O_s[(0, h)], r0.O_l[(0, h)]
        np.testing.assert_allclose(r1.O[(0, h)], a * Os + (1 - a) * Ol, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(r0.O[(0, 0)], r0.O_l[(0, 0)], atol=0)
    np.testing.assert_allclose(r0.O[(0, 1)], r0.O_s[(0, 1)], atol=0)


def test_constant_values_give_constant_output():
    # both branches are row-stochastic maps of V, so V == 1 gives O == 1
    rng = np.random.default_rng(8)
    N, d = 300, 16
    Q, K = rng.standard_normal((1, 1, N, d)), rng.standard_normal((1, 1, N, d))
    V = np.ones((1, 1, N, d))
    r = orc.forward(Q, K, V, _rand(d, d), _rand(d, d), [0.37], 0.2, 0.2)
    np.testing.assert_allclose(r.O[(0, 0)], 1.0, rtol=1e-13)


# --------------------------------------------------------------- invariances

def test_key_offset_invariance():
    # K -> K + c*1: phi(K), Pc, the mask, the sparse softmax and O are unchanged
    rng = np.random.default_rng(21)
    N, d = 320, 16
    Q, K, V = (rng.standard_normal((1, 1, N, d)) for _ in range(3))
    Pq, Pk = np.eye(d) + 0.1 * _rand(d, d), np.eye(d) + 0.1 * _rand(d, d)
    r0 = orc.forward(Q, K, V, Pq, Pk, [0.4], 0.2, 0.2)
    r1 = orc.forward(Q, K + 1.75, V, Pq, Pk, [0.4], 0.2, 0.2)
    np.testing.assert_array_equal(r0.mask, r1.mask)
    np.testing.assert_allclose(r1.O[(0, 0)], r0.O[(0, 0)], rtol=1e-10, atol=1e-12)


def test_permutation_inside_blocks():
    rng = np.random.default_rng(22)
    N, d = 256, 16
    Q, K, V = (rng.standard_normal((1, 1, N, d)) for _ in range(3))
    r0 = orc.forward(Q, K, V, np.eye(d), np.eye(d), [0.6], 0.25, 0.25)
    # keys: permute tokens inside block 2 together with V -> O unchanged
    p = np.arange(N)
    p[128:192] = 128 + rng.permutation(64)
    r1 = orc.forward(Q, K[:, :, p], V[:, :, p], np.eye(d), np.eye(d), [0.6], 0.25, 0.25)
    np.testing.assert_allclose(r1.O[(0, 0)], r0.O[(0, 0)], rtol=1e-12, atol=1e-13)
    # queries: permute tokens inside block 1 -> O rows permuted the same way
    q = np.arange(N)
    q[64:128] = 64 + rng.permutation(64)
    r2 = orc.forward(Q[:, :, q], K, V, np.eye(d), np.eye(d), [0.6], 0.25, 0.25)
    np.testing.assert_allclose(r2.O[(0, 0)], r0.O[(0, 0)][q], rtol=1e-12, atol=1e-13)


def test_query_block_subset_matches_full_rows():
    rng = np.random.default_rng(23)
    N, d = 640, 16
    Q, K, V = (rng.standard_normal((1, 2, N, d)) for _ in range(3))
    full = orc.forward(Q, K, V, np.eye(d), np.eye(d), [0.5, 0.5], 0.2, 0.3)
    sub = orc.forward(Q, K, V, np.eye(d), np.eye(d), [0.5, 0.5], 0.2, 0.3,
                      query_blocks={(0, 1): [7, 2]}, heads=[(0, 1)])
    rows = orc.token_rows([2, 7], N)
    np.testing.assert_array_equal(sub.O[(0, 1)], full.O[(0, 1)][rows])


def test_empty_sets_give_zero_branches():
    rng = np.random.default_rng(24)
    N, d, Nb = 256, 16, 4
    Q, K, V = (rng.standard_normal((1, 1, N, d)) for _ in range(3))
    mask = np.full((1, 1, Nb, Nb), -1, dtype=np.int8)
    mask[0, 0, 0, 1] = 1          # row 0: one critical, no marginal
    mask[0, 0, 1, 2] = 0          # row 1: one marginal, no critical
    r = orc.forward(Q, K, V, np.eye(d), np.eye(d), [0.5], 0.25, 0.25, mask_in=mask)
    assert not r.O_l[(0, 0)][0:64].any()
    assert not r.O_s[(0, 0)][64:128].any()
    assert not r.O[(0, 0)][128:].any()     # rows 2, 3: everything negligible
