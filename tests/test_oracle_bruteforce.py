"""Scalar brute force of the whole forward pass on tiny inputs.

Pure Python loops over single elements, with no matrix product, no blocking and
no numpy inside the arithmetic: an independent re-derivation of every step
(router projection, pooling, compressed scores, ranking, masked softmax, linear
branch, mix) that the float64 oracle must match to 1e-12 relative.
"""

import functools
import math

import numpy as np
import pytest

import oracle as orc


def brute_head(Q, K, V, Pq, Pk, alpha, n_h, n_l, feature="softmax", Po=None):
    """One head, scalar loops. feature: "softmax" or "elu1" (x + 1 for x > 0,
    exp(x) otherwise); Po: None for the SLA2 mix with alpha, else the SLA
    output map, O[t][c] = O_s[t][c] + sum_a O_l[t][a] Po[a][c]."""
    N, d = len(Q), len(Q[0])
    Nb = (N + 63) // 64

    def project(X, P):
        return [[sum(X[t][a] * P[a][c] for a in range(d)) for c in range(d)] for t in range(N)]

    def pool(X):
        out = []
        for i in range(Nb):
            toks = range(64 * i, min(64 * i + 64, N))
            out.append([sum(X[t][c] for t in toks) / len(toks) for c in range(d)])
        return out

    qbar, kbar = pool(project(Q, Pq)), pool(project(K, Pk))
    s = [[sum(qbar[i][c] * kbar[j][c] for c in range(d)) / math.sqrt(d) for j in range(Nb)]
         for i in range(Nb)]
    cls = []
    for i in range(Nb):
        def before(a, b):
            if s[i][a] != s[i][b]:
                return -1 if s[i][a] > s[i][b] else 1
            return (a > b) - (a < b)
        order = sorted(range(Nb), key=functools.cmp_to_key(before))
        row = [0] * Nb
        for r, j in enumerate(order):
            row[j] = 1 if r < n_h else (-1 if r >= Nb - n_l else 0)
        cls.append(row)

    def softmax(x):
        m = max(x)
        e = [math.exp(v - m) for v in x]
        z = sum(e)
        return [v / z for v in e]

    def feat(x):
        if feature == "softmax":
            return softmax(x)
        return [v + 1.0 if v > 0 else math.exp(v) for v in x]

    fk = [feat(K[t]) for t in range(N)]
    O = []
    for t in range(N):
        i = t // 64
        crit = [u for u in range(N) if cls[i][u // 64] == 1]
        marg = [u for u in range(N) if cls[i][u // 64] == 0]
        os_ = [0.0] * d
        if crit:
            x = [sum(Q[t][c] * K[u][c] for c in range(d)) / math.sqrt(d) for u in crit]
            w = softmax(x)
            os_ = [sum(w[n] * V[u][c] for n, u in enumerate(crit)) for c in range(d)]
        ol = [0.0] * d
        if marg:
            fq = feat(Q[t])
            a = [sum(fq[c] * fk[u][c] for c in range(d)) for u in marg]
            z = sum(a)
            ol = [sum(a[n] * V[u][c] for n, u in enumerate(marg)) / z for c in range(d)]
        if Po is None:
            O.append([alpha * os_[c] + (1 - alpha) * ol[c] for c in range(d)])
        else:
            O.append([os_[c] + sum(ol[a] * Po[a][c] for a in range(d)) for c in range(d)])
    return cls, O


@pytest.mark.parametrize("N,d,kh,kl", [(64, 16, 1.0, 0.0), (100, 16, 0.5, 0.0),
                                       (192, 16, 0.34, 0.34), (256, 16, 0.25, 0.5),
                                       (64, 64, 0.0, 0.0), (100, 64, 0.5, 0.5),
                                       (192, 64, 0.34, 0.0), (256, 64, 0.25, 0.25)])
def test_oracle_matches_scalar_brute_force(N, d, kh, kl):
    rng = np.random.default_rng(N * 1000 + d)
    H = 2
    Q = rng.standard_normal((1, H, N, d))
    K = rng.standard_normal((1, H, N, d))
    V = rng.standard_normal((1, H, N, d))
    Pq = np.eye(d) + 0.3 * rng.standard_normal((d, d))   # non-symmetric learned routers
    Pk = np.eye(d) + 0.3 * rng.standard_normal((d, d))
    alpha = [0.35, 0.8]
    res = orc.forward(Q, K, V, Pq, Pk, alpha, kh, kl)
    n_h, n_l = res.n_h, res.n_l
    h = int(rng.integers(0, H))
    cls, O = brute_head(Q[0, h].tolist(), K[0, h].tolist(), V[0, h].tolist(),
                        Pq.tolist(), Pk.tolist(), alpha[h], n_h, n_l)
    np.testing.assert_array_equal(res.mask[0, h], np.array(cls, dtype=np.int8))
    O = np.array(O)
    err = np.abs(res.O[(0, h)] - O).sum() / np.abs(O).sum()
    assert err < 1e-12, err


@pytest.mark.parametrize("N,d,kh,kl,feature,sla1", [
    (100, 16, 0.5, 0.0, "elu1", False), (192, 16, 0.34, 0.34, "elu1", True),
    (256, 16, 0.25, 0.25, "softmax", True), (64, 64, 0.0, 0.0, "elu1", True),
    (100, 64, 0.5, 0.5, "elu1", False), (192, 64, 0.34, 0.0, "softmax", True)])
def test_variants_match_scalar_brute_force(N, d, kh, kl, feature, sla1):
    """The ELU+1 feature map and the SLA output fusion O = O_s + Proj(O_l),
    against the same scalar re-derivation."""
    rng = np.random.default_rng(N * 7 + d)
    H = 2
    Q = rng.standard_normal((1, H, N, d))
    K = rng.standard_normal((1, H, N, d))
    V = rng.standard_normal((1, H, N, d))
    Pq = np.eye(d) + 0.3 * rng.standard_normal((d, d))
    Pk = np.eye(d) + 0.3 * rng.standard_normal((d, d))
    Po = rng.standard_normal((H, d, d)) / np.sqrt(d) if sla1 else None  # per-head, non-symmetric
    alpha = [0.3, 0.6]
    res = orc.forward(Q, K, V, Pq, Pk, None if sla1 else alpha, kh, kl, feature=feature,
                      proj_o=Po)
    for h in range(H):
        cls, O = brute_head(Q[0, h].tolist(), K[0, h].tolist(), V[0, h].tolist(), Pq.tolist(),
                            Pk.tolist(), alpha[h], res.n_h, res.n_l, feature,
                            None if Po is None else Po[h].tolist())
        np.testing.assert_array_equal(res.mask[0, h], np.array(cls, dtype=np.int8))
        O = np.array(O)
        err = np.abs(res.O[(0, h)] - O).sum() / np.abs(O).sum()
        assert err < 1e-12, err
