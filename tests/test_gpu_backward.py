"""GPU parity of the SLA2 backward pass (sla_backward) against the float64
autograd oracle (oracle/backward.py), for the block mask the forward pass
computes (or an injected one), through the C ABI.

Bounds, per (batch, head), on rel-L1 = sum |x - y| / sum |y|: fp32 inputs 1e-4
(fp32 arithmetic over sums of at most a few thousand terms); bf16 inputs 1e-2,
the forward's bf16 bound (the linear branch's H_i and Z_i are the forward's
bf16 ones). dalpha to 1e-4 (fp32) or 1e-2 (bf16) relative.
"""

import numpy as np
import pytest
import torch

import sparse_linear_attention_block_amd as sla
from oracle import backward as ob
from parity_util import rel_l1, run_gpu
from workloads import CONFIGS, make_inputs

pytestmark = pytest.mark.gpu


def _flush(msg):
    print(msg, flush=True)


def _grad_out(x, seed):
    g = np.random.default_rng(seed).standard_normal(tuple(x.q.shape))
    return torch.from_numpy(g.astype(np.float32)).to(x.q.dtype)


def _check(x, tol, mask=None, seed=7):
    if mask is None:
        mask = run_gpu(x, debug=False)["mask"]
    dO = _grad_out(x, seed)
    ref = ob.backward(x.q, x.k, x.v, x.alpha, mask, dO)
    dQ, dK, dV, da = sla.backward(x.q.cuda(), x.k.cuda(), x.v.cuda(), x.alpha.cuda(),
                                  torch.from_numpy(np.ascontiguousarray(mask)).cuda(), dO.cuda())
    torch.cuda.synchronize()
    got = {"dQ": dQ.cpu().numpy(), "dK": dK.cpu().numpy(), "dV": dV.cpu().numpy()}
    worst = 0.0
    for name in ("dQ", "dK", "dV"):
        for b in range(x.B):
            for h in range(x.H):
                e = rel_l1(got[name][b, h], ref[name][b, h])
                worst = max(worst, e)
                assert e <= tol, (name, b, h, e)
    da = da.cpu().numpy().astype(np.float64)
    eda = float(np.abs(da - ref["dalpha"]).max() / max(1e-12, np.abs(ref["dalpha"]).max()))
    _flush(f"B={x.B} H={x.H} N={x.N} d={x.d} {x.q.dtype}: worst rel-L1 {worst:.2e}, dalpha {eda:.2e}")
    assert eda <= tol, eda


def test_fp32_tiny():
    _check(make_inputs(CONFIGS[1]), 1e-4)


@pytest.mark.parametrize("N", [64, 100, 1000])
def test_bf16_recipe(N):
    _check(make_inputs(CONFIGS[2], H=2, N=N), 1e-2)


def test_bf16_d64():
    cfg = CONFIGS[1]
    x = make_inputs(cfg, N=700)
    x.q, x.k, x.v = x.q.bfloat16(), x.k.bfloat16(), x.v.bfloat16()
    _check(x, 1e-2)


@pytest.mark.parametrize("kh,kl", [(1.0, 0.0), (0.0, 0.0), (0.0, 0.5), (0.5, 0.5)])
def test_degenerate_fractions(kh, kl):
    _check(make_inputs(CONFIGS[2], H=2, N=640, kh=kh, kl=kl), 1e-2)


def test_injected_mask_with_empty_rows():
    x = make_inputs(CONFIGS[2], H=2, N=700)
    Nb = 11
    rng = np.random.default_rng(8)
    mask = rng.choice(np.array([1, 0, -1], dtype=np.int8), size=(1, 2, Nb, Nb))
    mask[0, 0, 3] = -1      # a row with neither critical nor marginal blocks
    mask[0, 1, 5] = 0       # a row with no critical block
    mask[0, 1, 6] = 1       # a row with no marginal block
    mask[0, 0, :, 4] = 1    # a key block critical for every row
    _check(x, 1e-2, mask=mask)


def test_fp32_d128():
    cfg = CONFIGS[2]
    x = make_inputs(cfg, H=2, N=300)
    x.q, x.k, x.v = x.q.float(), x.k.float(), x.v.float()
    _check(x, 1e-4)


def test_full_size_sampled():
    """The Wan2.1-1.3B shape (B=1, H=12, N=32760) in the launch shape the
    benchmark times: dQ on sampled query blocks of three heads against the
    oracle's per-block gradient, and the sum of dV over the keys against its
    closed form, sum_t (alpha [t has a critical block] + (1 - alpha) [t has
    a marginal one]) dO[t], on every head."""
    cfg = CONFIGS[3]
    x = make_inputs(cfg)
    mask = run_gpu(x, debug=False)["mask"]
    dO = _grad_out(x, 11)
    dQ, dK, dV, da = sla.backward(x.q.cuda(), x.k.cuda(), x.v.cuda(), x.alpha.cuda(),
                                  torch.from_numpy(mask).cuda(), dO.cuda())
    torch.cuda.synchronize()
    dQ, dV = dQ.cpu().numpy(), dV.cpu().numpy().astype(np.float64)
    rng = np.random.default_rng(12)
    for h in (0, 5, 11):
        blocks = sorted(rng.choice(cfg.Nb, 3, replace=False).tolist()) + [cfg.Nb - 1]
        ref = ob.dq_rows(x.q, x.k, x.v, x.alpha, mask, dO, 0, h, blocks)
        for i, r in ref.items():
            e = rel_l1(dQ[0, h, 64 * i:64 * i + r.shape[0]], r)
            _flush(f"head {h} block {i}: dQ rel-L1 {e:.2e}")
            assert e <= 1e-2, (h, i, e)
    g = dO.double().numpy()
    al = x.alpha.double().numpy()
    for h in range(cfg.H):
        c = np.repeat((mask[0, h] == 1).any(axis=1), 64)[:x.N].astype(float)
        m = np.repeat((mask[0, h] == 0).any(axis=1), 64)[:x.N].astype(float)
        w = al[h] * c + (1 - al[h]) * m
        expect = (w[:, None] * g[0, h]).sum(axis=0)
        e = rel_l1(dV[0, h].sum(axis=0), expect)
        assert e <= 1e-3, (h, e)
    _flush(f"sum of dV over the keys matches its closed form on all {cfg.H} heads")


def test_bf16_batch_of_two():
    # the CFG-batch recipe (B = 2, per-head alpha): dalpha sums over the batch
    _check(make_inputs(CONFIGS[4], H=3, N=500), 1e-2)
