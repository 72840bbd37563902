"""GPU checks of the training pair through the C ABI: sla_forward_train /
sla1_forward_train give the same O and mask as sla_forward / sla1_forward, and
sla_backward_saved / sla1_backward_saved, reading the state the saving forward
left in the workspace, give the same gradients as sla_backward /
sla1_backward, which the backward tests hold to the float64 oracle. The two
paths run the same kernels on the same inputs (the saving forward's sparse
kernel is the instance the backward's own recompute runs), so every output is
compared for equality, bit for bit; one case is also held to the oracle
directly.
"""

import numpy as np
import pytest
import torch

import sparse_linear_attention_block_amd as sla
from oracle import backward as ob
from parity_util import rel_l1
from workloads import CONFIGS, make_inputs, make_proj_o

pytestmark = pytest.mark.gpu


def _flush(msg):
    print(msg, flush=True)


def _grad_out(x, seed):
    g = np.random.default_rng(seed).standard_normal(tuple(x.q.shape))
    return torch.from_numpy(g.astype(np.float32)).to(x.q.dtype).cuda()


def _pair(x, *, phi="softmax", linear="gemm", mask_in=None, proj_o=None, seed=11):
    """Forward and backward both ways; returns the saved-path outputs after
    asserting that they equal the plain ones."""
    q, k, v = x.q.cuda(), x.k.cuda(), x.v.cuda()
    pq, pk, al = x.proj_q.cuda(), x.proj_k.cuda(), x.alpha.cuda()
    dO = _grad_out(x, seed)
    if proj_o is None:
        o_ref, m_ref = sla.forward(q, k, v, pq, pk, al, x.kh, x.kl, mask_in, phi=phi, linear=linear)
        o, m, ws = sla.forward_train(q, k, v, pq, pk, al, x.kh, x.kl, mask_in, phi=phi, linear=linear)
        g_ref = sla.backward(q, k, v, al, m_ref, dO, phi=phi, linear=linear)
        g = sla.backward_saved(q, k, v, al, m, dO, ws, phi=phi, linear=linear)
    else:
        W = proj_o.cuda()  # no router: SLA compares the block means themselves
        o_ref, m_ref = sla.forward_sla1(q, k, v, W, x.kh, x.kl, mask_in, phi=phi, linear=linear)
        o, m, ws = sla.forward_sla1_train(q, k, v, W, x.kh, x.kl, mask_in, phi=phi, linear=linear)
        g_ref = sla.backward_sla1(q, k, v, W, m_ref, dO, phi=phi, linear=linear)
        g = sla.backward_sla1_saved(q, k, v, W, m, dO, ws, phi=phi, linear=linear)
    torch.cuda.synchronize()
    assert torch.equal(m, m_ref), "mask"
    assert torch.equal(o, o_ref), "O"
    for name, a, b in zip(("dQ", "dK", "dV", "dalpha" if proj_o is None else "dproj_o"), g, g_ref):
        assert torch.equal(a, b), name
    _flush(f"B={x.B} H={x.H} N={x.N} d={x.d} phi={phi} linear={linear} sla1={proj_o is not None}: "
           f"O, mask and every gradient equal")
    return m, dO, g


@pytest.mark.parametrize("N", [64, 100, 1000, 4096])
def test_sla2_recipe(N):
    _pair(make_inputs(CONFIGS[2], H=2, N=N))


def test_sla2_against_the_oracle():
    x = make_inputs(CONFIGS[2], H=2, N=1000)
    m, dO, (dQ, dK, dV, da) = _pair(x)
    ref = ob.backward(x.q, x.k, x.v, x.alpha, m.cpu().numpy(), dO.cpu())
    got = {"dQ": dQ.cpu().numpy(), "dK": dK.cpu().numpy(), "dV": dV.cpu().numpy()}
    for name in got:
        for h in range(x.H):
            e = rel_l1(got[name][0, h], ref[name][0, h])
            assert e <= 1e-2, (name, h, e)
    da = da.cpu().numpy().astype(np.float64)
    assert float(np.abs(da - ref["dalpha"]).max() / np.abs(ref["dalpha"]).max()) <= 1e-2


def test_sla2_elu1_chain_and_injected_mask():
    x = make_inputs(CONFIGS[2], H=2, N=700)
    Nb = (x.N + 63) // 64
    rng = np.random.default_rng(5)
    mk = rng.choice(np.array([1, 0, -1], dtype=np.int8), size=(x.B, x.H, Nb, Nb), p=[0.2, 0.5, 0.3])
    mk[0, 0, 3] = -1  # a row with no critical block
    mk[0, 1, 4] = 1   # a row with no marginal block
    _pair(x, phi="elu1", linear="chain", mask_in=torch.from_numpy(mk).cuda())


def test_sla1_per_head_map():
    cfg = CONFIGS[2]
    x = make_inputs(cfg, H=2, N=1000)
    _pair(x, proj_o=make_proj_o(cfg, H=2, per_head=True))


def test_sla1_shared_map_elu1():
    cfg = CONFIGS[2]
    x = make_inputs(cfg, H=2, N=333)
    _pair(x, proj_o=make_proj_o(cfg, H=2), phi="elu1")


def test_full_size_wan13b():
    """The 1.3B shape the benchmark times: both paths equal, and the saved path
    leaves the workspace ready for the next training forward."""
    cfg = CONFIGS[3]
    x = make_inputs(cfg)
    _pair(x)
