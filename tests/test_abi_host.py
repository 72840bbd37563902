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
    (dict(elu=True), B.SLA_ERR_WORKSPACE),    # elu + 1 is built: valid up to the workspace
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


def _bwd1(p, Q=0x10000, K=0x10000, V=0x10000, W=0x10000, m=0x10000, dO=0x10000, dQ=0x10000,
          dK=0x10000, dV=0x10000, dW=0x10000, ws=None, wsb=0):
    lib = sla.load_library()
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.sla1_backward(ctypes.byref(p), vp(Q), vp(K), vp(V), vp(W), vp(m), vp(dO), vp(dQ), vp(dK),
                             vp(dV), vp(dW), vp(ws), ctypes.c_size_t(wsb), None)


@pytest.mark.parametrize("kw,code", [
    (dict(W=None), B.SLA_ERR_ARG),            # the output map is required
    (dict(dW=None), B.SLA_ERR_ARG),
    (dict(m=None), B.SLA_ERR_ARG),
    (dict(dW=0x10002), B.SLA_ERR_ARG),        # misaligned
    (dict(quant=True), B.SLA_ERR_UNSUPPORTED),
    (dict(), B.SLA_ERR_WORKSPACE),
    (dict(elu=True), B.SLA_ERR_WORKSPACE),
])
def test_sla1_backward_errors(kw, code):
    p = good()
    if kw.pop("quant", False):
        p.quant = B.SLA_QUANT_I8QK_F8PV
    if kw.pop("elu", False):
        p.phi = B.SLA_PHI_ELU1
    assert _bwd1(p, **kw) == code
    assert sla.load_library().sla_last_error()


def test_sla1_backward_workspace_adds_the_map_parts():
    lib = sla.load_library()
    p = sla.make_problem(1, 12, 32760, 128, "bf16", 0.05, 0.10)
    b2, b1 = ctypes.c_size_t(), ctypes.c_size_t()
    assert lib.sla_backward_workspace_bytes(ctypes.byref(p), ctypes.byref(b2)) == 0
    assert lib.sla1_backward_workspace_bytes(ctypes.byref(p), ctypes.byref(b1)) == 0
    # bf16 inputs: O_l in bf16, the 512 row-chunk parts of dW (float32), the range sums
    # (32 ranges, float64) and W as bf16 fragments for the MFMA kernels
    assert b1.value == b2.value + 12 * 32760 * 128 * 2 + 512 * 128 * 128 * 4 + 32 * 128 * 128 * 8 + 128 * 128 * 2
    # per-head maps: 512 // H chunk parts per head; float32 inputs: one part per query block
    ph = sla.make_problem(1, 12, 32760, 128, "bf16", 0.05, 0.10, proj_head_stride=128 * 128)
    bh2, bh1 = ctypes.c_size_t(), ctypes.c_size_t()
    assert lib.sla_backward_workspace_bytes(ctypes.byref(ph), ctypes.byref(bh2)) == 0
    assert lib.sla1_backward_workspace_bytes(ctypes.byref(ph), ctypes.byref(bh1)) == 0
    assert bh1.value == (bh2.value + 12 * 32760 * 128 * 2 + 12 * (512 // 12) * 128 * 128 * 4
                         + 12 * 32 * 128 * 128 * 8 + 12 * 128 * 128 * 2)
    f = sla.make_problem(1, 12, 32760, 128, "f32", 0.05, 0.10)
    f2, f1 = ctypes.c_size_t(), ctypes.c_size_t()
    assert lib.sla_backward_workspace_bytes(ctypes.byref(f), ctypes.byref(f2)) == 0
    assert lib.sla1_backward_workspace_bytes(ctypes.byref(f), ctypes.byref(f1)) == 0
    assert f1.value == f2.value + 12 * 512 * 128 * 128 * 4 + 32 * 128 * 128 * 8


def _train_call(name, p, ws=0x10000, wsb=0, **kw):
    """One call of the training pair with dummy aligned pointers (no device work:
    every case below fails its host checks first)."""
    lib = sla.load_library()
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    a = dict(Q=0x10000, K=0x10000, V=0x10000, x1=0x10000, x2=0x10000, x3=0x10000, x4=None, x5=0x10000,
             x6=0x10000, x7=0x10000, x8=0x10000)
    a.update(kw)
    fn = getattr(lib, name)
    if name.endswith("forward_train"):  # (p, Q, K, V, proj_q, proj_k, alpha | proj_o, mask_in, O, mask_out, ...)
        args = [a["Q"], a["K"], a["V"], a["x1"], a["x2"], a["x3"], a["x4"], a["x5"], a["x6"]]
    else:                               # (p, Q, K, V, alpha | proj_o, mask, dO, dQ, dK, dV, dalpha | dproj_o, ...)
        args = [a["Q"], a["K"], a["V"], a["x3"], a["x5"], a["x6"], a["x7"], a["x8"], a["x1"], a["x2"]]
    return fn(ctypes.byref(p), *[vp(x) for x in args], vp(ws), ctypes.c_size_t(wsb), None)


@pytest.mark.parametrize("name", ["sla_forward_train", "sla1_forward_train", "sla_backward_saved",
                                  "sla1_backward_saved"])
def test_training_pair_errors(name):
    lib = sla.load_library()
    p = good()
    assert _train_call(name, p) == B.SLA_ERR_WORKSPACE  # valid up to the workspace
    assert _train_call(name, p, x3=None) == B.SLA_ERR_ARG  # alpha / proj_o required
    f32 = good()
    f32.dtype = B.SLA_F32
    assert _train_call(name, f32) == B.SLA_ERR_UNSUPPORTED  # the bf16 MFMA path only
    q8 = good()
    q8.quant = B.SLA_QUANT_I8QK_F8PV
    assert _train_call(name, q8) == B.SLA_ERR_UNSUPPORTED
    assert lib.sla_last_error()
    if name.endswith("forward_train"):
        # the saving forward needs the backward's workspace, not the forward's
        fwd = ctypes.c_size_t()
        assert lib.sla_workspace_bytes(ctypes.byref(p), ctypes.byref(fwd)) == 0
        assert _train_call(name, p, wsb=fwd.value) == B.SLA_ERR_WORKSPACE


def test_backward_workspace_covers_the_forward():
    lib = sla.load_library()
    p = sla.make_problem(1, 12, 32760, 128, "bf16", 0.05, 0.10)
    fwd, bwd = ctypes.c_size_t(), ctypes.c_size_t()
    assert lib.sla_workspace_bytes(ctypes.byref(p), ctypes.byref(fwd)) == 0
    assert lib.sla_backward_workspace_bytes(ctypes.byref(p), ctypes.byref(bwd)) == 0
    # the forward's regions plus lse, D_t, dH_i per query block, their total and the partials
    Nb, NN = 512, 128 * 128 + 128
    assert bwd.value >= fwd.value + 12 * Nb * NN * 4 and bwd.value % 256 == 0


# ---- the Python binding's argument checks (host tensors; require_device=False
# lets every other rule be exercised without a GPU)

def _fwd_tensors(B=1, H=2, N=100, d=64, dtype=None):
    import torch
    dt = dtype or torch.bfloat16
    q = torch.zeros(B, H, N, d, dtype=dt)
    Nb = (N + 63) // 64
    return dict(q=q, k=q.clone(), v=q.clone(), proj_q=torch.eye(d), proj_k=torch.eye(d),
                alpha=torch.full((H,), 0.5), mask_in=torch.zeros(B, H, Nb, Nb, dtype=torch.int8),
                out=torch.empty_like(q), mask_out=torch.empty(B, H, Nb, Nb, dtype=torch.int8))


def test_binding_accepts_valid_arguments():
    import torch
    t = _fwd_tensors()
    assert B.validate_forward_args(**t, require_device=False) == 0
    t["proj_q"] = torch.zeros(2, 64, 64)
    t["proj_k"] = torch.zeros(2, 64, 64)
    assert B.validate_forward_args(**t, require_device=False) == 64 * 64
    t = _fwd_tensors()
    t.update(proj_q=None, proj_k=None, alpha=None, proj_o=torch.eye(64))
    assert B.validate_forward_args(**t, require_device=False) == 0


def _bad(change):
    import torch
    t = _fwd_tensors()
    change(t, torch)
    return t


@pytest.mark.parametrize("change,match", [
    (lambda t, torch: t.update(k=torch.zeros(1, 2, 99, 64, dtype=torch.bfloat16)), "share one"),
    (lambda t, torch: t.update(v=t["v"].float()), "bfloat16 or all float32"),
    (lambda t, torch: t.update(q=t["q"].half(), k=t["k"].half(), v=t["v"].half(),
                               out=t["out"].half()), "bfloat16 or all float32"),
    (lambda t, torch: t.update(q=t["q"].transpose(2, 3).contiguous().transpose(2, 3)), "contiguous"),
    (lambda t, torch: t.update(proj_q=torch.eye(32), proj_k=torch.eye(32)), r"\[d, d\] or \[H, d, d\]"),
    (lambda t, torch: t.update(proj_q=torch.zeros(3, 64, 64), proj_k=torch.zeros(3, 64, 64)),
     r"\[d, d\] or \[H, d, d\]"),
    (lambda t, torch: t.update(proj_q=torch.eye(64, dtype=torch.float64)), "float32"),
    (lambda t, torch: t.update(proj_k=torch.zeros(2, 64, 64)), "one shape"),
    (lambda t, torch: t.update(proj_k=None), "both given"),
    (lambda t, torch: t.update(alpha=torch.full((3,), 0.5)), "alpha"),
    (lambda t, torch: t.update(alpha=torch.full((2,), 0.5, dtype=torch.float64)), "alpha"),
    (lambda t, torch: t.update(alpha=None), "alpha"),
    (lambda t, torch: t.update(proj_o=torch.eye(64), proj_q=torch.zeros(2, 64, 64),
                               proj_k=torch.zeros(2, 64, 64)), "head stride"),
    (lambda t, torch: t.update(proj_o=torch.eye(48)), r"\[d, d\] or \[H, d, d\]"),
    (lambda t, torch: t.update(mask_in=torch.zeros(1, 2, 2, 3, dtype=torch.int8)), "mask_in"),
    (lambda t, torch: t.update(mask_in=torch.zeros(1, 2, 2, 2, dtype=torch.int32)), "mask_in"),
    (lambda t, torch: t.update(out=torch.empty(1, 2, 100, 64)), "out"),
    (lambda t, torch: t.update(out=torch.empty(1, 2, 99, 64, dtype=torch.bfloat16)), "out"),
    (lambda t, torch: t.update(mask_out=torch.empty(1, 2, 2, 2, dtype=torch.int16)), "mask_out"),
    (lambda t, torch: t.update(mask_out=torch.empty(1, 2, 3, 2, dtype=torch.int8)), "mask_out"),
    (lambda t, torch: t.update(alpha=torch.full((2,), 0.5, device="meta")), "not on q's device"),
    (lambda t, torch: t.update(proj_q=torch.eye(64, device="meta")), "not on q's device"),
    (lambda t, torch: t.update(out=torch.empty(1, 2, 100, 64, dtype=torch.bfloat16, device="meta")),
     "not on q's device"),
])
def test_binding_rejects(change, match):
    with pytest.raises(ValueError, match=match):
        B.validate_forward_args(**_bad(change), require_device=False)


def test_binding_requires_device_tensors():
    with pytest.raises(ValueError, match="device tensors"):
        B.validate_forward_args(**_fwd_tensors())
    import torch
    t = _fwd_tensors()
    with pytest.raises(ValueError, match="device tensors"):
        sla.backward(t["q"], t["k"], t["v"], t["alpha"], t["mask_in"], t["q"])
    with pytest.raises(ValueError, match="device tensors"):
        sla.forward(t["q"], t["k"], t["v"], t["proj_q"], t["proj_k"], t["alpha"], 0.25, 0.25)


def test_noalloc_scratch_size_matches_header():
    text = open(os.path.join(ROOT, "include", "sla.h")).read()
    m = re.search(r"#define SLA_NOALLOC_SCRATCH_BYTES \((\d+)u \* 1024u \* 1024u\)", text)
    assert m and int(m.group(1)) * 2 ** 20 == sla.noalloc_scratch_bytes()


def test_noalloc_rejects_problems_beyond_its_scratch():
    """Host-only: the size check returns before any device work."""
    lib = sla.load_library()
    p = sla.make_problem(1, 12, 32760, 128, "bf16", 0.05, 0.10)
    assert sla.workspace_bytes(p) > sla.noalloc_scratch_bytes()
    fake = ctypes.c_void_p(0x10000)
    rc = lib.sla_forward_noalloc(ctypes.byref(p), fake, fake, fake, fake, fake, fake, None, fake, fake, None)
    assert rc == B.SLA_ERR_WORKSPACE
    assert b"scratch" in lib.sla_last_error()
    bad = sla.make_problem(1, 12, 100, 96, "bf16", 0.05, 0.10)   # d = 96 is not built
    assert lib.sla_forward_noalloc(ctypes.byref(bad), fake, fake, fake, fake, fake, fake, None, fake, fake,
                                   None) == B.SLA_ERR_UNSUPPORTED


def test_linear_sums_field():
    lib = sla.load_library()
    n = ctypes.c_size_t()
    g = sla.make_problem(1, 12, 32760, 128, "bf16", 0.05, 0.10)
    c = sla.make_problem(1, 12, 32760, 128, "bf16", 0.05, 0.10, linear="chain")
    assert lib.sla_workspace_bytes(ctypes.byref(g), ctypes.byref(n)) == 0
    ng = n.value
    assert lib.sla_workspace_bytes(ctypes.byref(c), ctypes.byref(n)) == 0
    # the chain's per-row lists and counts (the indicator and its product still have their regions)
    assert n.value >= ng + 12 * 512 * 512 * 2 + 12 * 512 * 4
    bad = sla.make_problem(1, 2, 1000, 64, "bf16", 0.2, 0.2)
    bad.linear_sums = 7
    assert lib.sla_workspace_bytes(ctypes.byref(bad), ctypes.byref(n)) == B.SLA_ERR_ARG
    f32 = sla.make_problem(1, 2, 1000, 64, "f32", 0.2, 0.2, linear="chain")
    assert lib.sla_workspace_bytes(ctypes.byref(f32), ctypes.byref(n)) == B.SLA_ERR_UNSUPPORTED
    ok = sla.make_problem(1, 2, 1216 * 64, 64, "bf16", 0.01, 0.01, linear="chain")
    assert lib.sla_workspace_bytes(ctypes.byref(ok), ctypes.byref(n)) == 0
    big = sla.make_problem(1, 2, 1216 * 64 + 1, 64, "bf16", 0.01, 0.01, linear="chain")
    assert lib.sla_workspace_bytes(ctypes.byref(big), ctypes.byref(n)) == B.SLA_ERR_UNSUPPORTED
    with pytest.raises(ValueError):
        sla.make_problem(1, 2, 100, 64, "bf16", 0.2, 0.2, linear="lut")
