"""GPU parity of the backward passes (sla_backward for SLA2, sla1_backward
for the SLA fusion O = O_s + O_l W, either feature map) against the float64
autograd oracle (oracle/backward.py), for the block mask the forward pass
computes (or an injected one), through the C ABI.

Bounds, per (batch, head), on rel-L1 = sum |x - y| / sum |y|: fp32 inputs 1e-4
(fp32 arithmetic over sums of at most a few thousand terms); bf16 inputs 1e-2,
the forward's bf16 bound (the linear branch's H_i and Z_i are the forward's
bf16 ones). dalpha to 1e-4 (fp32) or 1e-2 (bf16) relative; dW to the same
rel-L1 bounds. For bf16 inputs without the output map the products run on
bf16 MFMA: P, dS, phi and the linear-branch gradients enter them rounded to
bf16 (relative 2^-9), so the closed form of the sum of dV over the keys, whose
error is that of the few dominant weights of each row, is held to 3e-3.
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
    worst = 0.0
    for h in range(cfg.H):
        c = np.repeat((mask[0, h] == 1).any(axis=1), 64)[:x.N].astype(float)
        m = np.repeat((mask[0, h] == 0).any(axis=1), 64)[:x.N].astype(float)
        w = al[h] * c + (1 - al[h]) * m
        expect = (w[:, None] * g[0, h]).sum(axis=0)
        e = rel_l1(dV[0, h].sum(axis=0), expect)
        worst = max(worst, e)
        assert e <= 3e-3, (h, e)
    _flush(f"sum of dV over the keys matches its closed form on all {cfg.H} heads (worst {worst:.2e})")


def test_largest_supported_block_count():
    """Nb = 4096, the largest block count the library takes (N = 262107, a
    ragged last block of 27 tokens), one head at d = 128: dQ on query blocks at
    both ends and on both sides of index 2048 against the oracle's per-block
    gradient, and the sum of dV over the keys against its closed form (as in
    the full-size test above); the chunked dK/dV work runs over 4096 key blocks
    with 1024 partial slots."""
    from workloads.configs import WorkloadConfig
    N = 4096 * 64 - 37
    cfg = WorkloadConfig(14, "max_nb_bwd", 1, 1, N, 128, None, "bf16", 0.01, 0.05, "learned",
                         ("const", 0.6), False, 85, qk="normal")
    x = make_inputs(cfg)
    assert cfg.Nb == 4096
    mask = run_gpu(x, debug=False)["mask"]
    dO = _grad_out(x, 13)
    dQ, dK, dV, da = sla.backward(x.q.cuda(), x.k.cuda(), x.v.cuda(), x.alpha.cuda(),
                                  torch.from_numpy(mask).cuda(), dO.cuda())
    torch.cuda.synchronize()
    dQ, dV = dQ.cpu().numpy(), dV.cpu().numpy().astype(np.float64)
    assert np.isfinite(dK.cpu().numpy()).all()
    ref = ob.dq_rows(x.q, x.k, x.v, x.alpha, mask, dO, 0, 0, [0, 1, 2047, 2048, 4095])
    for i, r in ref.items():
        e = rel_l1(dQ[0, 0, 64 * i:64 * i + r.shape[0]], r)
        _flush(f"max Nb block {i}: dQ rel-L1 {e:.2e}")
        assert e <= 1e-2, (i, e)
    al = float(x.alpha.double()[0])
    c = np.repeat((mask[0, 0] == 1).any(axis=1), 64)[:N].astype(float)
    m = np.repeat((mask[0, 0] == 0).any(axis=1), 64)[:N].astype(float)
    expect = ((al * c + (1 - al) * m)[:, None] * dO.double().numpy()[0, 0]).sum(axis=0)
    e = rel_l1(dV[0, 0].sum(axis=0), expect)
    _flush(f"max Nb: sum of dV over the keys against its closed form {e:.2e}")
    assert e <= 3e-3, e


def test_bf16_batch_of_two():
    # the CFG-batch recipe (B = 2, per-head alpha): dalpha sums over the batch
    _check(make_inputs(CONFIGS[4], H=3, N=500), 1e-2)


# ---- ELU+1 and the SLA formulation O = O_s + O_l W (sla1_backward)

def _check_sla1(x, tol, W, phi="softmax", mask=None, seed=21):
    if mask is None:
        mask = run_gpu(x, debug=False, proj_o=W, router=False, phi=phi)["mask"]
    dO = _grad_out(x, seed)
    ref = ob.backward(x.q, x.k, x.v, None, mask, dO, phi=phi, proj_o=W)
    dQ, dK, dV, dW = sla.backward_sla1(x.q.cuda(), x.k.cuda(), x.v.cuda(), W.cuda(),
                                       torch.from_numpy(np.ascontiguousarray(mask)).cuda(), dO.cuda(), phi=phi)
    torch.cuda.synchronize()
    got = {"dQ": dQ.cpu().numpy(), "dK": dK.cpu().numpy(), "dV": dV.cpu().numpy()}
    worst = 0.0
    for name in ("dQ", "dK", "dV"):
        for b in range(x.B):
            for h in range(x.H):
                e = rel_l1(got[name][b, h], ref[name][b, h])
                worst = max(worst, e)
                assert e <= tol, (name, b, h, e)
    eW = rel_l1(dW.cpu().numpy(), ref["dproj_o"])
    _flush(f"SLA {phi} W{list(W.shape)} B={x.B} H={x.H} N={x.N} d={x.d} {x.q.dtype}: worst rel-L1 {worst:.2e}, "
           f"dW {eW:.2e}")
    assert eW <= tol, eW


def _proj(d, H=None, seed=5):
    rng = np.random.default_rng(seed)
    shape = (d, d) if H is None else (H, d, d)
    return torch.from_numpy((np.eye(d) + 0.3 * rng.standard_normal(shape) / np.sqrt(d)).astype(np.float32))


@pytest.mark.parametrize("N", [100, 1000])
def test_elu1_sla2_bf16(N):
    x = make_inputs(CONFIGS[2], H=2, N=N)
    mask = run_gpu(x, debug=False, phi="elu1")["mask"]
    dO = _grad_out(x, 9)
    ref = ob.backward(x.q, x.k, x.v, x.alpha, mask, dO, phi="elu1")
    dQ, dK, dV, da = sla.backward(x.q.cuda(), x.k.cuda(), x.v.cuda(), x.alpha.cuda(),
                                  torch.from_numpy(mask).cuda(), dO.cuda(), phi="elu1")
    torch.cuda.synchronize()
    for name, t in (("dQ", dQ), ("dK", dK), ("dV", dV)):
        for h in range(2):
            e = rel_l1(t.cpu().numpy()[0, h], ref[name][0, h])
            assert e <= 1e-2, (name, h, e)
    eda = float(np.abs(da.cpu().numpy() - ref["dalpha"]).max() / np.abs(ref["dalpha"]).max())
    _flush(f"SLA2 elu1 N={N}: dalpha {eda:.2e}")
    assert eda <= 1e-2


def test_sla1_fp32_tiny():
    x = make_inputs(CONFIGS[1])
    _check_sla1(x, 1e-4, _proj(64))
    _check_sla1(x, 1e-4, _proj(64, H=2), phi="elu1")


@pytest.mark.parametrize("phi", ["softmax", "elu1"])
@pytest.mark.parametrize("per_head", [False, True])
def test_sla1_bf16(phi, per_head):
    x = make_inputs(CONFIGS[2], H=3, N=1000)
    _check_sla1(x, 1e-2, _proj(128, H=3 if per_head else None), phi=phi)


def test_sla1_batch_of_two_injected_mask():
    # dW sums over the batch (and the heads, W shared); rows with empty sets
    x = make_inputs(CONFIGS[4], H=2, N=500)
    Nb = 8
    rng = np.random.default_rng(22)
    mask = rng.choice(np.array([1, 0, -1], dtype=np.int8), size=(2, 2, Nb, Nb))
    mask[0, 0, 2] = -1
    mask[1, 1, 3] = 0
    mask[1, 0, 4] = 1
    _check_sla1(x, 1e-2, _proj(128), mask=mask)


@pytest.mark.parametrize("N,per_head", [(20, True), (20, False), (37, True), (100, False)])
def test_sla1_bf16_steps_across_pairs(N, per_head):
    # the bf16 dW product walks the rows of every (batch, head) pair that shares a
    # map in steps of 32: with N < 32 one step spans several pairs; B = 2
    x = make_inputs(CONFIGS[4], H=3, N=N)
    Nb = (N + 63) // 64
    # one block per row: make it marginal, so that O_l and dW are not zero
    mask = np.zeros((x.B, x.H, Nb, Nb), dtype=np.int8) if Nb == 1 else None
    _check_sla1(x, 1e-2, _proj(128, H=3 if per_head else None), mask=mask)


def test_sla1_bf16_d64_batch_of_two():
    x = make_inputs(CONFIGS[1], B=2, N=700)
    x.q, x.k, x.v = x.q.bfloat16(), x.k.bfloat16(), x.v.bfloat16()
    _check_sla1(x, 1e-2, _proj(64, H=x.H))
    _check_sla1(x, 1e-2, _proj(64), phi="elu1")


def test_sla1_fp32_d128():
    x = make_inputs(CONFIGS[2], H=2, N=300)
    x.q, x.k, x.v = x.q.float(), x.k.float(), x.v.float()
    _check_sla1(x, 1e-4, _proj(128, H=2), phi="elu1")
