"""The seeded synthetic inputs: shapes, determinism and calibration to the pages."""

import json
import os

import numpy as np
import torch

from workloads import CONFIGS, make_inputs, sincos_posemb

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_shapes_and_dtypes_small():
    x = make_inputs(CONFIGS[1])
    assert x.q.shape == (1, 2, 1024, 64) and x.q.dtype == torch.float32
    assert torch.equal(x.proj_q, torch.eye(64)) and torch.all(x.alpha == 0.5)
    y = make_inputs(CONFIGS[2], H=2, N=1000)
    assert y.q.shape == (1, 2, 1000, 128) and y.q.dtype == torch.bfloat16
    assert y.alpha.shape == (2,) and float(y.alpha.min()) >= 0.2 and float(y.alpha.max()) <= 0.8
    assert not torch.equal(y.proj_q, torch.eye(128))


def test_deterministic_and_sliceable():
    a = make_inputs(CONFIGS[4], B=1, H=2, N=300)
    b = make_inputs(CONFIGS[4], B=2, H=3, N=300)
    assert torch.equal(a.q, b.q[:1, :2]) and torch.equal(a.v, b.v[:1, :2])
    c = make_inputs(CONFIGS[4], B=1, H=2, N=300)
    assert torch.equal(a.k, c.k)


def test_posemb_norm():
    p = sincos_posemb((3, 5, 7), 128)
    np.testing.assert_allclose((p ** 2).sum(axis=1), 64.0, rtol=1e-12)


def test_attention_peakedness_matches_pages_fig1():
    """Dense softmax attention of the mid-size workload has about the share of
    large (> 1/N) and tiny (< 1/(100N)) weights the pages report for Wan2.1."""
    g = json.load(open(os.path.join(GOLDEN, "fig1_weight_distribution.json")))
    x = make_inputs(CONFIGS[2], H=4)
    N, d = x.N, x.d
    big, tiny = [], []
    rng = np.random.default_rng(0)
    for h in range(4):
        q = x.q[0, h].double().numpy()
        k = x.k[0, h].double().numpy()
        rows = rng.choice(N, 128, replace=False)
        S = q[rows] @ k.T / np.sqrt(d)
        W = np.exp(S - S.max(axis=1, keepdims=True))
        W /= W.sum(axis=1, keepdims=True)
        big.append((W > 1.0 / N).mean())
        tiny.append((W < 1.0 / (100 * N)).mean())
    big, tiny = float(np.mean(big)), float(np.mean(tiny))
    assert abs(big - g["critical_above_mean_1_over_N"]) < 0.04, big
    assert abs(tiny - g["negligible_below_1_over_100N"]) < 0.10, tiny
