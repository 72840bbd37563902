"""GPU parity of the chain form of the marginal sums (sla_problem.linear_sums
= SLA_LINEAR_CHAIN): each query block's H_i, Z_i taken from the previous
block's by adding the h_j, z_j of blocks that became marginal and subtracting
those that stopped being marginal (SLA paper summary, Eq. 3; SLA explainer,
section 2.3). The linear branch O_l (debug output) and O are held to the
oracle at the bf16 bar with the oracle's mask injected, and O_l to the
indicator-product form at rel-L1 2e-3 (the two round float32 sums of the same
bf16 terms in different orders before one bf16 rounding of H_i)."""

import numpy as np
import pytest
import torch

import oracle as orc
from parity_util import (BF16_MAX_ABS, BF16_REL_L1, compare_masks, rel_l1, run_gpu,
                         sample_query_blocks)
import sparse_linear_attention_block_amd as sla
from workloads import CONFIGS, make_inputs

pytestmark = pytest.mark.gpu

FORMS_REL_L1 = 2e-3


def _flush(msg):
    print(msg, flush=True)


def _run(x, mask, linear, quant=False, phi="softmax"):
    q, k, v = x.q.cuda(), x.k.cuda(), x.v.cuda()
    mi = torch.from_numpy(np.ascontiguousarray(mask)).cuda()
    o, _, dbg = sla.forward(q, k, v, x.proj_q.cuda(), x.proj_k.cuda(), x.alpha.cuda(), x.kh, x.kl,
                            mask_in=mi, debug=True, quant=quant, phi=phi, linear=linear)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), dbg["o_l"].cpu().numpy()


def _check(x, mask, heads=None, qblocks=None, quant=False, phi="softmax"):
    heads = heads or [(b, h) for b in range(x.B) for h in range(x.H)]
    sub = orc.forward(x.q, x.k, x.v, x.proj_q, x.proj_k, x.alpha, x.kh, x.kl, mask_in=mask, heads=heads,
                      query_blocks=qblocks, feature=phi)
    oc, lc = _run(x, mask, "chain", quant, phi)
    og, lg = _run(x, mask, "gemm", quant, phi)
    for (b, h) in heads:
        rows = np.arange(x.N) if qblocks is None else orc.token_rows(qblocks[(b, h)], x.N)
        e_l = rel_l1(lc[b, h][rows], sub.O_l[(b, h)])
        m_l = float(np.abs(lc[b, h][rows] - sub.O_l[(b, h)]).max())
        e_o = rel_l1(oc[b, h][rows], sub.O[(b, h)])
        e_f = rel_l1(lc[b, h], lg[b, h])
        _flush(f"head {(b, h)}: chain O_l {e_l:.2e} / {m_l:.2e}, O {e_o:.2e}; chain vs product O_l {e_f:.2e}")
        assert e_l <= BF16_REL_L1 and m_l <= BF16_MAX_ABS, ("O_l", b, h, e_l, m_l)
        assert e_f <= FORMS_REL_L1, ("forms", b, h, e_f)
        if not quant:
            assert e_o <= BF16_REL_L1, ("O", b, h, e_o)


@pytest.mark.parametrize("N", [100, 1000, 4096])
def test_chain_recipe(N):
    x = make_inputs(CONFIGS[2], H=2, N=N)
    ref = orc.forward(x.q, x.k, x.v, x.proj_q, x.proj_k, x.alpha, x.kh, x.kl, compute_outputs=False)
    _check(x, ref.mask)


def test_chain_injected_edges():
    """Rows with nothing marginal, everything marginal, equal to the row before,
    all classes flipped from the row before; Nb = 20 > 16 segments of 2 rows."""
    x = make_inputs(CONFIGS[2], H=2, N=1250)
    Nb = 20
    rng = np.random.default_rng(31)
    mask = rng.choice([1, 0, -1], size=(1, 2, Nb, Nb), p=[0.2, 0.6, 0.2]).astype(np.int8)
    mask[0, 0, 3] = 1
    mask[0, 0, 4] = 0
    mask[0, 0, 5] = mask[0, 0, 4]
    mask[0, 1, 7] = np.where(mask[0, 1, 6] == 0, 1, 0)
    mask[0, 1, 19] = -1
    _check(x, mask)


def test_chain_elu1_d64():
    cfg = CONFIGS[1]
    x = make_inputs(cfg, N=3000)
    x.q, x.k, x.v = x.q.bfloat16(), x.k.bfloat16(), x.v.bfloat16()
    ref = orc.forward(x.q, x.k, x.v, x.proj_q, x.proj_k, x.alpha, x.kh, x.kl, compute_outputs=False)
    _check(x, ref.mask, phi="elu1")


@pytest.mark.timeout(600)
def test_chain_14b_shape_sampled():
    """The 14B-720P shape (B=1, H=40, N=75600, Nb=1182) in 8-bit mode, the
    configuration the chain is aimed at: the mask the GPU computes (exact
    against the oracle on every row), then O_l on sampled query blocks of three
    heads."""
    cfg = CONFIGS[5]
    x = make_inputs(cfg)
    ref = orc.forward(x.q, x.k, x.v, x.proj_q, x.proj_k, x.alpha, x.kh, x.kl, compute_outputs=False)
    g = run_gpu(x, debug=False, quant=True)
    exact, excused, bad = compare_masks(g["mask"], ref.mask, ref.logits, ref.n_h, ref.n_l)
    assert not bad, bad[:10]
    heads = [(0, 0), (0, 19), (0, cfg.H - 1)]
    qb = {hh: sample_query_blocks(cfg.Nb, 6, 41 * hh[1] + 3) for hh in heads}
    _check(x, ref.mask, heads=heads, qblocks=qb, quant=True)
