"""The C-ABI library on the host: exported symbols, block counts, workspace
sizing and every argument error path (all return before any device work, so
these run without a GPU)."""

import ctypes
import math
import os
import re

import pytest

import oracle as orc
import sparse_linear_attention_block_amd as sla
from sparse_linear_attention_block_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "sla.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sla1?_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = sla.load_library()
    names = _declared_functions()
    assert {"sla_forward", "sla_forward_debug", "sla_workspace_bytes", "sla_block_counts",
            "sla_status_str", "sla_last_error", "sla_version", "sla1_forward",
            "sla1_forward_debug"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert lib.sla_version() >> 16 == 1


@pytest.mark.parametrize("N", [1, 63, 64, 65, 1000, 1024, 8192, 32760, 75600, 262144])
@pytest.mark.parametrize("kh,kl", [(0.05, 0.10), (0.03, 0.10), (0.25, 0.25), (0.0, 0.0),
                                   (1.0, 0.0), (0.29, 0.0), (0.0, 1.0)])
def test_block_counts_match_oracle(N, kh, kl):
    Nb = orc.num_blocks(N)
    try:
        ref = orc.block_counts(Nb, kh, kl)
    except ValueError:
        with pytest.raises(sla.SLAError) as e:
            sla.block_counts(N, kh, kl)
        assert e.value.status == B.SLA_ERR_ARG
        return
    assert sla.block_counts(N, kh, kl) == (Nb, *ref)


def test_workspace_bytes_scale_and_alignment():
    small = sla.workspace_bytes(sla.make_problem(1, 2, 1024, 64, "f32", 0.25, 0.25))
    big = sla.workspace_bytes(sla.make_problem(1, 12, 32760, 128, "bf16", 0.05, 0.10))
    assert 0 < small < big and small % 256 == 0 and big % 256 == 0


def _fwd(p, Q=0x10000, K=0x10000, V=0x10000, pq=0x10000, pk=0x10000, al=0x10000, mi=None,
         O=0x10000, mo=0x10000, ws=0x10000, wsb=0):
    lib = sla.load_library()
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.sla_forward(ctypes.byref(p) if p is not None else None, vp(Q), vp(K), vp(V),
                           vp(pq), vp(pk), vp(al), vp(mi), vp(O), vp(mo), vp(ws),
                           ctypes.c_size_t(wsb), None)


def good():
    return sla.make_problem(1, 2, 1000, 128, "bf16", 0.05, 0.10)


@pytest.mark.parametrize("mutate,code", [
    (lambda p: setattr(p, "B", 0), B.SLA_ERR_ARG),
    (lambda p: setattr(p, "N", -5), B.SLA_ERR_ARG),
    (lambda p: setattr(p, "dtype", 7), B.SLA_ERR_ARG),
    (lambda p: setattr(p, "kh", float("nan")), B.SLA_ERR_ARG),
    (lambda p: setattr(p, "kl", 1.5), B.SLA_ERR_ARG),
    (lambda p: (setattr(p, "kh", 0.6), setattr(p, "kl", 0.5)), B.SLA_ERR_ARG),
    (lambda p: setattr(p, "phi", 7), B.SLA_ERR_ARG),
    (lambda p: setattr(p, "proj_head_stride", 5), B.SLA_ERR_ARG),
    (lambda p: setattr(p, "d", 96), B.SLA_ERR_UNSUPPORTED),
    (lambda p: (setattr(p, "dtype", B.SLA_F32), setattr(p, "quant", 1)), B.SLA_ERR_UNSUPPORTED),
    (lambda p: setattr(p, "N", 4096 * 64 + 1), B.SLA_ERR_UNSUPPORTED),
])
def test_problem_errors(mutate, code):
    p = good()
    mutate(p)
    assert _fwd(p) == code
    n = ctypes.c_size_t()
    assert sla.load_library().sla_workspace_bytes(ctypes.byref(p), ctypes.byref(n)) == code
    assert sla.load_library().sla_last_error()


def test_null_problem():
    assert _fwd(None) == B.SLA_ERR_ARG


@pytest.mark.parametrize("kw,code", [
    (dict(Q=None), B.SLA_ERR_ARG),
    (dict(alpha_none=True), B.SLA_ERR_ARG),
    (dict(O=None), B.SLA_ERR_ARG),
    (dict(pq=None), B.SLA_ERR_ARG),          # one router matrix without the other
    (dict(pk=None), B.SLA_ERR_ARG),
    (dict(pq=None, pk=None), B.SLA_ERR_WORKSPACE),  # no router is valid: the workspace check follows
    (dict(mo=None), B.SLA_ERR_ARG),          # mask_out needed without mask_in
    (dict(Q=0x10008), B.SLA_ERR_ARG),        # misaligned
    (dict(al=0x10002), B.SLA_ERR_ARG),
    (dict(ws=None), B.SLA_ERR_WORKSPACE),
    (dict(ws=0x10080, wsb=1 << 40), B.SLA_ERR_WORKSPACE),  # misaligned workspace
    (dict(wsb=100), B.SLA_ERR_WORKSPACE),    # too small
])
def test_pointer_and_workspace_errors(kw, code):
    if kw.pop("alpha_none", False):
        kw["al"] = None
    assert _fwd(good(), **kw) == code
    assert sla.load_library().sla_last_error()


def test_status_strings():
    lib = sla.load_library()
    for c in (0, -1, -2, -3, -4):
        assert lib.sla_status_str(c)
    assert b"unknown" in lib.sla_status_str(42)


def _fwd1(p, Q=0x10000, K=0x10000, V=0x10000, pq=None, pk=None, po=0x10000, mi=None,
          O=0x10000, mo=0x10000, ws=0x10000, wsb=0):
    lib = sla.load_library()
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.sla1_forward(ctypes.byref(p), vp(Q), vp(K), vp(V), vp(pq), vp(pk), vp(po), vp(mi),
                            vp(O), vp(mo), vp(ws), ctypes.c_size_t(wsb), None)


@pytest.mark.parametrize("kw,code", [
    (dict(po=None), B.SLA_ERR_ARG),          # the output map is required
    (dict(po=0x10002), B.SLA_ERR_ARG),       # misaligned
    (dict(pq=0x10000), B.SLA_ERR_ARG),       # one router matrix without the other
    (dict(quant=True), B.SLA_ERR_UNSUPPORTED),
    (dict(), B.SLA_ERR_WORKSPACE),           # valid up to the workspace; no alpha needed
    (dict(pq=0x10000, pk=0x10000), B.SLA_ERR_WORKSPACE),
])
def test_sla1_errors(kw, code):
    p = good()
    if kw.pop("quant", False):
        p.quant = B.SLA_QUANT_I8QK_F8PV
    assert _fwd1(p, **kw) == code
    assert sla.load_library().sla_last_error()


def test_feature_map_does_not_change_sizes():
    a = sla.make_problem(1, 12, 32760, 128, "bf16", 0.05, 0.10)
    b = sla.make_problem(1, 12, 32760, 128, "bf16", 0.05, 0.10, phi="elu1")
    assert sla.workspace_bytes(a) == sla.workspace_bytes(b)
    with pytest.raises(ValueError):
        sla.make_problem(1, 1, 64, 64, "bf16", 0.5, 0.0, phi="relu")


def _stk(lg=0x10000, rows=4, cols=64, k=3.0, tau=1e-3, out=0x10000, lam=None):
    lib = sla.load_library()
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.sla_soft_topk(vp(lg), rows, cols, k, tau, vp(out), vp(lam), None)


@pytest.mark.parametrize("kw", [
    dict(lg=None), dict(out=None), dict(lg=0x10004), dict(out=0x10002), dict(lam=0x10001),
    dict(rows=0), dict(cols=0), dict(cols=4097), dict(k=-1.0), dict(k=64.5),
    dict(k=float("nan")), dict(tau=0.0), dict(tau=-1.0), dict(tau=float("inf")),
])
def test_soft_topk_argument_errors(kw):
    assert _stk(**kw) == B.SLA_ERR_ARG
    assert sla.load_library().sla_last_error()


def _bwd(p, Q=0x10000, K=0x10000, V=0x10000, al=0x10000, m=0x10000, dO=0x10000, dQ=0x10000,
         dK=0x10000, dV=0x10000, da=0x10000, ws=0x10000, wsb=0):
    lib = sla.load_library()
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.sla_backward(ctypes.byref(p), vp(Q), vp(K), vp(V), vp(al), vp(m), vp(dO), vp(dQ), vp(dK),
                            vp(dV), vp(da), vp(ws), ctypes.c_size_t(wsb), None)


@pytest.mark.parametrize("kw,code", [
    (dict(m=None), B.SLA_ERR_ARG),            # the forward's mask is required
    (dict(dO=None), B.SLA_ERR_ARG),
    (dict(dK=None), B.SLA_ERR_ARG),
    (dict(da=None), B.SLA_ERR_ARG),
    (dict(dQ=0x10004), B.SLA_ERR_ARG),        # misaligned
    (dict(al=0x10001), B.SLA_ERR_ARG),
    (dict(quant=True), B.SLA_ERR_UNSUPPORTED),
    (dict(elu=True), B.SLA_ERR_UNSUPPORTED),
    (dict(), B.SLA_ERR_WORKSPACE),            # valid up to the workspace
    (dict(ws=0x10080, wsb=1 << 40), B.SLA_ERR_WORKSPACE),
])
def test_backward_errors(kw, code):
    p = good()
    if kw.pop("quant", False):
        p.quant = B.SLA_QUANT_I8QK_F8PV
    if kw.pop("elu", False):
        p.phi = B.SLA_PHI_ELU1
    assert _bwd(p, **kw) == code
    assert sla.load_library().sla_last_error()


def test_backward_workspace_covers_the_forward():
    lib = sla.load_library()
    p = sla.make_problem(1, 12, 32760, 128, "bf16", 0.05, 0.10)
    fwd, bwd = ctypes.c_size_t(), ctypes.c_size_t()
    assert lib.sla_workspace_bytes(ctypes.byref(p), ctypes.byref(fwd)) == 0
    assert lib.sla_backward_workspace_bytes(ctypes.byref(p), ctypes.byref(bwd)) == 0
    # the forward's regions plus lse, D_t, dH_i per query block, their total and the partials
    Nb, NN = 512, 128 * 128 + 128
    assert bwd.value >= fwd.value + 12 * Nb * NN * 4 and bwd.value % 256 == 0
