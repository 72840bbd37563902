"""GPU parity of the SLA formulation and the ELU+1 feature map (through the C ABI).

sla1_forward fuses the branches as O = O_s + Proj(O_l) (SLA paper summary,
section 4, step 4); sla_problem.phi = SLA_PHI_ELU1 makes the linear branch use
phi = elu + 1 (Eq. 3's symbol list, Table 2). Both are held to the same bars
as the SLA2 path, against the float64 oracle run with the same options:
the mask exactly (near-ties excused), and, with the oracle's mask injected,
O, O_s and the linear term (Proj(O_l) for SLA, O_l for SLA2) per head at
fp32 rel-L1 <= 1e-5, or bf16 rel-L1 <= 1e-2 and max-abs <= 2e-2.
"""

import numpy as np
import pytest

import oracle as orc
from parity_util import (BF16_MAX_ABS, BF16_REL_L1, F32_REL_L1, compare_masks, rel_l1,
                         run_gpu, sample_query_blocks)
from workloads import CONFIGS, make_inputs, make_proj_o

pytestmark = pytest.mark.gpu


def _flush(msg):
    print(msg, flush=True)


def _check(x, tol_rel, tol_abs=None, phi="softmax", proj_o=None, router=True):
    pq, pk = (x.proj_q, x.proj_k) if router else (None, None)
    _flush(f"B={x.B} H={x.H} N={x.N} d={x.d} kh={x.kh} kl={x.kl} phi={phi} "
           f"sla1={proj_o is not None} router={router}")
    ref = orc.forward(x.q, x.k, x.v, pq, pk, x.alpha, x.kh, x.kl, feature=phi, proj_o=proj_o)
    g = run_gpu(x, phi=phi, proj_o=proj_o, router=router)
    np.testing.assert_allclose(g["pooled_q"], ref.pooled_q, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(g["logits"], ref.logits, rtol=1e-10, atol=1e-11)
    exact, excused, bad = compare_masks(g["mask"], ref.mask, ref.logits, ref.n_h, ref.n_l)
    _flush(f"mask rows exact={exact} near-tie={excused} bad={len(bad)}")
    assert not bad, bad[:10]
    gi = run_gpu(x, mask_in=ref.mask, phi=phi, proj_o=proj_o, router=router)
    lin = "O_lp" if proj_o is not None else "O_l"
    worst = 0.0
    for b in range(x.B):
        for h in range(x.H):
            for name, key in (("O", "O"), ("O_s", "o_s"), (lin, "o_l")):
                r = getattr(ref, name)[(b, h)]
                e = rel_l1(gi[key][b, h], r)
                worst = max(worst, e)
                assert e <= tol_rel, (name, b, h, e)
                if tol_abs is not None:
                    m = float(np.abs(gi[key][b, h] - r).max())
                    assert m <= tol_abs, (name, b, h, m)
    _flush(f"worst rel-L1 {worst:.2e}")
    return ref, g, gi


@pytest.mark.parametrize("phi", ["softmax", "elu1"])
def test_fp32_sla1(phi):
    x = make_inputs(CONFIGS[1])
    _check(x, F32_REL_L1, phi=phi, proj_o=make_proj_o(CONFIGS[1]), router=False)


def test_fp32_elu1_sla2_mix():
    x = make_inputs(CONFIGS[1])
    _check(x, F32_REL_L1, phi="elu1")


@pytest.mark.parametrize("N", [100, 1000, 4096])
@pytest.mark.parametrize("phi", ["softmax", "elu1"])
def test_bf16_sla1_small(N, phi):
    x = make_inputs(CONFIGS[2], H=2, N=N)
    _check(x, BF16_REL_L1, BF16_MAX_ABS, phi=phi, proj_o=make_proj_o(CONFIGS[2]), router=False)


@pytest.mark.parametrize("N", [100, 4096])
def test_bf16_elu1_sla2_mix(N):
    x = make_inputs(CONFIGS[2], H=2, N=N)
    _check(x, BF16_REL_L1, BF16_MAX_ABS, phi="elu1")


def test_bf16_sla1_per_head_with_router():
    cfg = CONFIGS[2]
    x = make_inputs(cfg, H=3, N=1500)
    # one stride for all three matrices: the router becomes [H, d, d] too
    x.proj_q = x.proj_q.expand(3, -1, -1).contiguous()
    x.proj_k = x.proj_k.expand(3, -1, -1).contiguous()
    _check(x, BF16_REL_L1, BF16_MAX_ABS, phi="elu1", proj_o=make_proj_o(cfg, H=3, per_head=True))


def test_d64_sla1():
    cfg = CONFIGS[1]
    x = make_inputs(cfg)
    x.q, x.k, x.v = x.q.bfloat16(), x.k.bfloat16(), x.v.bfloat16()
    _check(x, BF16_REL_L1, BF16_MAX_ABS, phi="elu1", proj_o=make_proj_o(cfg), router=False)


@pytest.mark.parametrize("kh,kl", [(1.0, 0.0), (0.0, 0.0), (0.0, 0.5), (0.3, 0.2)])
def test_degenerate_fractions_sla1(kh, kl):
    x = make_inputs(CONFIGS[2], H=2, N=640, kh=kh, kl=kl)
    _check(x, BF16_REL_L1, BF16_MAX_ABS, phi="elu1", proj_o=make_proj_o(CONFIGS[2]), router=False)


def test_single_ragged_block_sla1():
    x = make_inputs(CONFIGS[2], H=2, N=37, kh=0.5, kl=0.0)
    _check(x, BF16_REL_L1, BF16_MAX_ABS, proj_o=make_proj_o(CONFIGS[2]), router=False)


def test_constant_values_give_one_plus_column_sums():
    # V == 1: both branches give ones, so O = 1 + column sums of Proj (in bf16)
    cfg = CONFIGS[2]
    x = make_inputs(cfg, H=2, N=1000, kh=0.2, kl=0.2)
    x.v.fill_(1.0)
    W = make_proj_o(cfg)
    g = run_gpu(x, phi="elu1", proj_o=W, router=False, debug=False)
    expect = 1.0 + W.double().sum(dim=0).numpy()
    e = rel_l1(g["O"], np.broadcast_to(expect, g["O"].shape))
    _flush(f"constant V: rel-L1 {e:.2e}")
    assert e <= BF16_REL_L1


def test_full_size_sla1_elu1_sampled():
    """The Wan2.1-1.3B shape (B=1, H=12, N=32760, kh = 5%, kl = 10%) in the
    launch shape the benchmark times for the SLA formulation: the mask on every
    row, outputs on sampled query blocks of sampled heads."""
    cfg = CONFIGS[3]
    x = make_inputs(cfg)
    W = make_proj_o(cfg)
    heads = [(0, 0), (0, cfg.H - 1), (0, cfg.H // 2)]
    ref = orc.forward(x.q, x.k, x.v, None, None, None, x.kh, x.kl, compute_outputs=False,
                      feature="elu1", proj_o=W)
    g = run_gpu(x, phi="elu1", proj_o=W, router=False, debug=False)
    exact, excused, bad = compare_masks(g["mask"], ref.mask, ref.logits, ref.n_h, ref.n_l)
    _flush(f"mask rows exact={exact} near-tie={excused} bad={len(bad)}")
    assert not bad, bad[:10]
    gi = run_gpu(x, mask_in=ref.mask, phi="elu1", proj_o=W, router=False, debug=True)
    qb = {hh: sample_query_blocks(cfg.Nb, 6, 31 * hh[1] + 5) for hh in heads}
    sub = orc.forward(x.q, x.k, x.v, None, None, None, x.kh, x.kl, mask_in=ref.mask, heads=heads,
                      query_blocks=qb, feature="elu1", proj_o=W)
    for (b, h) in heads:
        rows = orc.token_rows(qb[(b, h)], x.N)
        for name, key in (("O", "O"), ("O_s", "o_s"), ("O_lp", "o_l")):
            r = getattr(sub, name)[(b, h)]
            gg = gi[key][b, h][rows]
            e = rel_l1(gg, r)
            m = float(np.abs(gg - r).max())
            _flush(f"head {(b, h)} {name}: rel-L1 {e:.2e} max-abs {m:.2e}")
            assert e <= BF16_REL_L1 and m <= BF16_MAX_ABS, (name, b, h, e, m)
