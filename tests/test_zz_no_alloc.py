"""sla_forward_noalloc (the entry point for callers that cannot allocate)
against sla_forward on the GPU, through the C ABI.

Two calls in a row on one GPU, the second with a smaller problem (so the
scratch holds the first call's larger layout when the second starts): each
output and mask must equal sla_forward's bit for bit (the same kernels on the
same inputs), and the output must meet the bf16 bar against the float64 oracle.
"""

import numpy as np
import pytest
import torch

import oracle as orc
import sparse_linear_attention_block_amd as sla
from parity_util import BF16_MAX_ABS, BF16_REL_L1, rel_l1
from workloads import CONFIGS, make_inputs

pytestmark = pytest.mark.gpu


def _noalloc_vs_forward(x, quant=False):
    dev = torch.device("cuda:0")
    q, k, v = x.q.to(dev), x.k.to(dev), x.v.to(dev)
    pq, pk, al = x.proj_q.to(dev), x.proj_k.to(dev), x.alpha.to(dev)
    B, H, N, d = q.shape
    Nb = (N + 63) // 64
    ref_o, ref_m = sla.forward(q, k, v, pq, pk, al, x.kh, x.kl, quant=quant)
    out = torch.full_like(q, float("nan"))
    mask = torch.full((B, H, Nb, Nb), 7, dtype=torch.int8, device=dev)
    o, m = sla.forward_noalloc(q, k, v, pq, pk, al, x.kh, x.kl, out, mask_out=mask, quant=quant)
    torch.cuda.synchronize()
    assert o.data_ptr() == out.data_ptr() and m.data_ptr() == mask.data_ptr()
    assert torch.equal(m, ref_m), "mask differs from sla_forward's"
    assert torch.equal(o.view(torch.int16), ref_o.view(torch.int16)), "O differs from sla_forward's"
    return o.float().cpu().numpy(), m.cpu().numpy()


def test_noalloc_two_calls_second_smaller():
    big = make_inputs(CONFIGS[2], H=4, N=4096)
    small = make_inputs(CONFIGS[2], H=2, N=1000)     # ragged tail of 40 tokens
    for x in (big, small):
        print(f"noalloc: H={x.H} N={x.N}", flush=True)
        o, m = _noalloc_vs_forward(x)
        heads = [(0, 0), (0, x.H - 1)]
        ref = orc.forward(x.q, x.k, x.v, x.proj_q, x.proj_k, x.alpha, x.kh, x.kl, mask_in=m, heads=heads)
        for (b, h) in heads:
            e = rel_l1(o[b, h], ref.O[(b, h)])
            assert e <= BF16_REL_L1 and np.abs(o[b, h] - ref.O[(b, h)]).max() <= BF16_MAX_ABS, (b, h, e)


def test_noalloc_8bit_after_bf16():
    x = make_inputs(CONFIGS[5], H=2, N=2000)
    print(f"noalloc 8-bit: H={x.H} N={x.N}", flush=True)
    _noalloc_vs_forward(x, quant=True)
