"""ctypes binding of libsla.so (argument marshalling only).

Every step of the forward pass runs in the HIP kernels behind the C ABI of
include/sla.h; PyTorch only supplies device memory and the current stream.
There is no fallback: without the built library every call raises.
"""

import ctypes
import os
from typing import Optional

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsla.so")

SLA_OK, SLA_ERR_ARG, SLA_ERR_UNSUPPORTED, SLA_ERR_WORKSPACE, SLA_ERR_HIP = 0, -1, -2, -3, -4
SLA_F32, SLA_BF16 = 0, 1
SLA_QUANT_NONE, SLA_QUANT_I8QK_F8PV = 0, 1
SLA_PHI_SOFTMAX, SLA_PHI_ELU1 = 0, 1
_PHI = {"softmax": SLA_PHI_SOFTMAX, "elu1": SLA_PHI_ELU1}
SLA_LINEAR_GEMM, SLA_LINEAR_CHAIN = 0, 1
_LINEAR = {"gemm": SLA_LINEAR_GEMM, "chain": SLA_LINEAR_CHAIN}


class Problem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("N", ctypes.c_int32),
                ("d", ctypes.c_int32), ("dtype", ctypes.c_int32), ("quant", ctypes.c_int32),
                ("proj_head_stride", ctypes.c_int32), ("phi", ctypes.c_int32),
                ("kh", ctypes.c_double), ("kl", ctypes.c_double), ("linear_sums", ctypes.c_int32)]


class Debug(ctypes.Structure):
    _fields_ = [("pooled_q", ctypes.c_void_p), ("pooled_k", ctypes.c_void_p),
                ("logits", ctypes.c_void_p), ("o_s", ctypes.c_void_p), ("o_l", ctypes.c_void_p),
                ("events", ctypes.c_void_p * 6)]


class SLAError(RuntimeError):
    def __init__(self, status: int, text: str):
        super().__init__(text)
        self.status = status


_lib = None

_FWD_ARGS = [ctypes.POINTER(Problem), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
             ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
             ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Loads libsla.so once; raises ImportError if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python -m sparse_linear_attention_block_amd.build`")
    lib = ctypes.CDLL(path)
    lib.sla_block_counts.argtypes = [ctypes.POINTER(Problem), ctypes.POINTER(ctypes.c_int32),
                                     ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32)]
    lib.sla_block_counts.restype = ctypes.c_int
    lib.sla_workspace_bytes.argtypes = [ctypes.POINTER(Problem), ctypes.POINTER(ctypes.c_size_t)]
    lib.sla_workspace_bytes.restype = ctypes.c_int
    lib.sla_forward.argtypes = _FWD_ARGS
    lib.sla_forward.restype = ctypes.c_int
    lib.sla_forward_debug.argtypes = _FWD_ARGS + [ctypes.POINTER(Debug)]
    lib.sla_forward_debug.restype = ctypes.c_int
    # the SLA formulation: proj_o in alpha's place
    lib.sla1_forward.argtypes = _FWD_ARGS
    lib.sla1_forward.restype = ctypes.c_int
    lib.sla1_forward_debug.argtypes = _FWD_ARGS + [ctypes.POINTER(Debug)]
    lib.sla1_forward_debug.restype = ctypes.c_int
    lib.sla_forward_noalloc.argtypes = _FWD_ARGS[:10] + [ctypes.c_void_p]
    lib.sla_forward_noalloc.restype = ctypes.c_int
    lib.sla_backward_workspace_bytes.argtypes = [ctypes.POINTER(Problem), ctypes.POINTER(ctypes.c_size_t)]
    lib.sla_backward_workspace_bytes.restype = ctypes.c_int
    lib.sla_backward.argtypes = [ctypes.POINTER(Problem)] + [ctypes.c_void_p] * 10 + [ctypes.c_void_p, ctypes.c_size_t,
                                                                                      ctypes.c_void_p]
    lib.sla_backward.restype = ctypes.c_int
    lib.sla1_backward_workspace_bytes.argtypes = [ctypes.POINTER(Problem), ctypes.POINTER(ctypes.c_size_t)]
    lib.sla1_backward_workspace_bytes.restype = ctypes.c_int
    lib.sla1_backward.argtypes = lib.sla_backward.argtypes
    lib.sla1_backward.restype = ctypes.c_int
    # the training pair: a forward that keeps the backward's inputs in the workspace
    for fn in (lib.sla_forward_train, lib.sla1_forward_train):
        fn.argtypes = _FWD_ARGS
        fn.restype = ctypes.c_int
    for fn in (lib.sla_backward_saved, lib.sla1_backward_saved):
        fn.argtypes = lib.sla_backward.argtypes
        fn.restype = ctypes.c_int
    lib.sla_soft_topk.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_double,
                                  ctypes.c_double, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.sla_soft_topk.restype = ctypes.c_int
    lib.sla_status_str.argtypes = [ctypes.c_int]
    lib.sla_status_str.restype = ctypes.c_char_p
    lib.sla_last_error.argtypes = []
    lib.sla_last_error.restype = ctypes.c_char_p
    lib.sla_version.argtypes = []
    lib.sla_version.restype = ctypes.c_int
    _lib = lib
    return lib


def _check(rc: int) -> None:
    if rc != SLA_OK:
        lib = load_library()
        raise SLAError(rc, f"{lib.sla_status_str(rc).decode()}: {lib.sla_last_error().decode()}")


def make_problem(B: int, H: int, N: int, d: int, dtype: str, kh: float, kl: float,
                 quant: bool = False, proj_head_stride: int = 0, phi: str = "softmax",
                 linear: str = "gemm") -> Problem:
    if phi not in _PHI:
        raise ValueError(f"phi must be one of {sorted(_PHI)}")
    if linear not in _LINEAR:
        raise ValueError(f"linear must be one of {sorted(_LINEAR)}")
    return Problem(B, H, N, d, SLA_BF16 if dtype in ("bf16", torch.bfloat16) else SLA_F32,
                   SLA_QUANT_I8QK_F8PV if quant else SLA_QUANT_NONE, proj_head_stride, _PHI[phi],
                   float(kh), float(kl), _LINEAR[linear])


def block_counts(N: int, kh: float, kl: float, *, B: int = 1, H: int = 1, d: int = 128,
                 dtype: str = "bf16"):
    """(Nb, n_h, n_l) as the library computes them (host only)."""
    lib = load_library()
    p = make_problem(B, H, N, d, dtype, kh, kl)
    nb, nh, nl = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    _check(lib.sla_block_counts(ctypes.byref(p), ctypes.byref(nb), ctypes.byref(nh), ctypes.byref(nl)))
    return nb.value, nh.value, nl.value


def workspace_bytes(p: Problem) -> int:
    lib = load_library()
    n = ctypes.c_size_t()
    _check(lib.sla_workspace_bytes(ctypes.byref(p), ctypes.byref(n)))
    return n.value


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _same_device(name, t, dev):
    if t is not None and t.device != dev:
        raise ValueError(f"{name} is on {t.device}, not on q's device {dev}")


def _check_router(name, t, H, d):
    if t.dtype != torch.float32:
        raise ValueError(f"{name} must be float32")
    if tuple(t.shape) not in ((d, d), (H, d, d)):
        raise ValueError(f"{name} must be [d, d] or [H, d, d] = [{d}, {d}] or [{H}, {d}, {d}] "
                         f"(got {list(t.shape)})")


def validate_forward_args(q, k, v, proj_q=None, proj_k=None, alpha=None, proj_o=None,
                          mask_in=None, out=None, mask_out=None, require_device=True) -> int:
    """Checks every tensor argument of a forward call before any pointer
    reaches the library (a host tensor, or one of the wrong shape, would be
    read out of bounds by the kernels). Returns the router / output-map head
    stride in elements (0 or d*d); raises ValueError otherwise.
    require_device=False skips only the "is a GPU tensor" test, so that the
    remaining rules can be exercised on host tensors."""
    if q.dim() != 4 or tuple(k.shape) != tuple(q.shape) or tuple(v.shape) != tuple(q.shape):
        raise ValueError("q, k, v must share one [B, H, N, d] shape")
    if require_device and not q.is_cuda:
        raise ValueError("q, k, v must be device tensors")
    if q.dtype not in (torch.bfloat16, torch.float32) or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must all be bfloat16 or all float32")
    B, H, N, d = q.shape
    Nb = (N + 63) // 64
    dev = q.device
    for name, t in (("k", k), ("v", v), ("proj_q", proj_q), ("proj_k", proj_k), ("alpha", alpha),
                    ("proj_o", proj_o), ("mask_in", mask_in), ("out", out), ("mask_out", mask_out)):
        _same_device(name, t, dev)
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    hs = 0
    if (proj_q is None) != (proj_k is None):
        raise ValueError("proj_q and proj_k are both given or both None")
    if proj_q is not None:
        _check_router("proj_q", proj_q, H, d)
        _check_router("proj_k", proj_k, H, d)
        if proj_k.shape != proj_q.shape:
            raise ValueError("proj_q and proj_k must have one shape")
        hs = d * d if proj_q.dim() == 3 else 0
    if proj_o is not None:
        _check_router("proj_o", proj_o, H, d)
        ohs = d * d if proj_o.dim() == 3 else 0
        if proj_q is not None and ohs != hs:
            raise ValueError("proj_q, proj_k and proj_o share one head stride: all [d, d] or all [H, d, d]")
        hs = ohs
    else:
        if alpha is None or alpha.dtype != torch.float32 or alpha.numel() != H:
            raise ValueError("alpha must be float32 with H entries")
    if mask_in is not None and (mask_in.dtype != torch.int8 or tuple(mask_in.shape) != (B, H, Nb, Nb)):
        raise ValueError("mask_in must be int8 [B, H, Nb, Nb]")
    if out is not None and (out.dtype != q.dtype or tuple(out.shape) != tuple(q.shape)
                            or not out.is_contiguous()):
        raise ValueError("out must be a contiguous tensor of q's dtype and shape")
    if mask_out is not None and (mask_out.dtype != torch.int8 or tuple(mask_out.shape) != (B, H, Nb, Nb)
                                 or not mask_out.is_contiguous()):
        raise ValueError("mask_out must be a contiguous int8 [B, H, Nb, Nb] tensor")
    return hs


def _run(q, k, v, proj_q, proj_k, alpha, proj_o, kh, kl, mask_in, quant, out, mask_out,
         workspace, debug, phi, linear="gemm", train=False):
    lib = load_library()
    hs = validate_forward_args(q, k, v, proj_q, proj_k, alpha, proj_o, mask_in, out, mask_out)
    B, H, N, d = q.shape
    Nb = (N + 63) // 64
    dev = q.device
    if proj_q is not None:
        proj_q, proj_k = proj_q.contiguous(), proj_k.contiguous()
    if proj_o is not None:
        proj_o = proj_o.contiguous()
    else:
        alpha = alpha.contiguous()
    if mask_in is not None:
        mask_in = mask_in.contiguous()
    if workspace is not None and (workspace.device != dev or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous tensor on q's device")
    p = make_problem(B, H, N, d, "bf16" if q.dtype == torch.bfloat16 else "f32", kh, kl,
                     quant, hs, phi, linear)
    if train:
        need = ctypes.c_size_t()
        size_fn = lib.sla_backward_workspace_bytes if proj_o is None else lib.sla1_backward_workspace_bytes
        _check(size_fn(ctypes.byref(p), ctypes.byref(need)))
        need = need.value
    else:
        need = workspace_bytes(p)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    if out is None:
        out = torch.empty_like(q)
    if mask_in is None and mask_out is None:
        mask_out = torch.empty((B, H, Nb, Nb), dtype=torch.int8, device=dev)
    dbg = None
    dbg_t = {}
    if debug:
        if mask_in is None:
            dbg_t["pooled_q"] = torch.empty((B, H, Nb, d), dtype=torch.float64, device=dev)
            dbg_t["pooled_k"] = torch.empty((B, H, Nb, d), dtype=torch.float64, device=dev)
            dbg_t["logits"] = torch.empty((B, H, Nb, Nb), dtype=torch.float64, device=dev)
        dbg_t["o_s"] = torch.empty((B, H, N, d), dtype=torch.float32, device=dev)
        dbg_t["o_l"] = torch.empty((B, H, N, d), dtype=torch.float32, device=dev)
        dbg = Debug(*[_ptr(dbg_t.get(n)) for n in ("pooled_q", "pooled_k", "logits", "o_s", "o_l")])
    with torch.cuda.device(dev):
        stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
        args = [ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(proj_q), _ptr(proj_k),
                _ptr(alpha if proj_o is None else proj_o), _ptr(mask_in), _ptr(out), _ptr(mask_out),
                _ptr(workspace), ctypes.c_size_t(workspace.numel() * workspace.element_size()), stream]
        if train:
            rc = (lib.sla_forward_train if proj_o is None else lib.sla1_forward_train)(*args)
        elif proj_o is None:
            rc = lib.sla_forward_debug(*args, ctypes.byref(dbg)) if debug else lib.sla_forward(*args)
        else:
            rc = lib.sla1_forward_debug(*args, ctypes.byref(dbg)) if debug else lib.sla1_forward(*args)
    _check(rc)
    mask = mask_out if mask_out is not None else mask_in
    if train:
        return out, mask, workspace
    if debug:
        return out, mask, dbg_t
    return out, mask


def forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
            proj_q: Optional[torch.Tensor], proj_k: Optional[torch.Tensor], alpha: torch.Tensor,
            kh: float, kl: float, mask_in: Optional[torch.Tensor] = None, *,
            quant: bool = False, out: Optional[torch.Tensor] = None,
            mask_out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
            debug: bool = False, phi: str = "softmax", linear: str = "gemm"):
    """SLA2 forward on the GPU (sla_forward): returns (O, mask) or (O, mask, debug dict).

    q, k, v: [B, H, N, d] contiguous bf16 or float32 device tensors.
    proj_q, proj_k: float32 [d, d] or [H, d, d], or both None (no router projection).
    alpha: float32 [H]. mask_in: optional int8 [B, H, Nb, Nb] in {1, 0, -1}.
    phi: the linear branch's feature map, "softmax" or "elu1".
    linear: how the marginal sums are formed, "gemm" (the indicator product)
    or "chain" (row-to-row updates).
    """
    return _run(q, k, v, proj_q, proj_k, alpha, None, kh, kl, mask_in, quant, out, mask_out,
                workspace, debug, phi, linear)


def forward_train(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                  proj_q: Optional[torch.Tensor], proj_k: Optional[torch.Tensor], alpha: torch.Tensor,
                  kh: float, kl: float, mask_in: Optional[torch.Tensor] = None, *,
                  out: Optional[torch.Tensor] = None, mask_out: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None, phi: str = "softmax", linear: str = "gemm"):
    """SLA2 forward that keeps the backward pass's inputs (sla_forward_train):
    returns (O, mask, workspace). Pass the three, unchanged, with the same q, k,
    v and alpha to backward_saved. bf16 inputs only."""
    return _run(q, k, v, proj_q, proj_k, alpha, None, kh, kl, mask_in, False, out, mask_out,
                workspace, False, phi, linear, train=True)


def forward_sla1_train(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, proj_o: torch.Tensor,
                       kh: float, kl: float, mask_in: Optional[torch.Tensor] = None, *,
                       proj_q: Optional[torch.Tensor] = None, proj_k: Optional[torch.Tensor] = None,
                       out: Optional[torch.Tensor] = None, mask_out: Optional[torch.Tensor] = None,
                       workspace: Optional[torch.Tensor] = None, phi: str = "softmax",
                       linear: str = "gemm"):
    """SLA forward that keeps the backward pass's inputs (sla1_forward_train):
    returns (O, mask, workspace) for backward_sla1_saved. bf16 inputs only."""
    if proj_o is None:
        raise ValueError("proj_o is required")
    return _run(q, k, v, proj_q, proj_k, None, proj_o, kh, kl, mask_in, False, out, mask_out,
                workspace, False, phi, linear, train=True)


def noalloc_scratch_bytes() -> int:
    """Bytes of the per-GPU scratch that forward_noalloc uses (SLA_NOALLOC_SCRATCH_BYTES)."""
    return 160 * 1024 * 1024


def forward_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                    proj_q: Optional[torch.Tensor], proj_k: Optional[torch.Tensor], alpha: torch.Tensor,
                    kh: float, kl: float, out: torch.Tensor, mask_in: Optional[torch.Tensor] = None,
                    mask_out: Optional[torch.Tensor] = None, *, quant: bool = False,
                    phi: str = "softmax"):
    """SLA2 forward without a workspace (sla_forward_noalloc): the library's
    per-GPU scratch holds the intermediates, so this call allocates nothing on
    the device. The caller passes the output `out` (q's dtype and shape) and,
    unless mask_in is given, `mask_out` (int8 [B, H, Nb, Nb]). Returns
    (out, mask). Calls that overlap on one GPU race on the shared scratch."""
    lib = load_library()
    validate_forward_args(q, k, v, proj_q, proj_k, alpha, None, mask_in, out, mask_out)
    if out is None or (mask_in is None and mask_out is None):
        raise ValueError("forward_noalloc needs out, and mask_out unless mask_in is given")
    for name, t in (("proj_q", proj_q), ("proj_k", proj_k), ("alpha", alpha), ("mask_in", mask_in)):
        if t is not None and not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous (this call may not copy)")
    B, H, N, d = q.shape
    hs = d * d if (proj_q is not None and proj_q.dim() == 3) else 0
    p = make_problem(B, H, N, d, "bf16" if q.dtype == torch.bfloat16 else "f32", kh, kl, quant, hs, phi)
    with torch.cuda.device(q.device):
        stream = ctypes.c_void_p(torch.cuda.current_stream(q.device).cuda_stream)
        rc = lib.sla_forward_noalloc(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(proj_q), _ptr(proj_k),
                                     _ptr(alpha), _ptr(mask_in), _ptr(out), _ptr(mask_out), stream)
    _check(rc)
    return out, (mask_out if mask_out is not None else mask_in)


def forward_sla1(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, proj_o: torch.Tensor,
                 kh: float, kl: float, mask_in: Optional[torch.Tensor] = None, *,
                 proj_q: Optional[torch.Tensor] = None, proj_k: Optional[torch.Tensor] = None,
                 out: Optional[torch.Tensor] = None, mask_out: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None, debug: bool = False,
                 phi: str = "softmax", linear: str = "gemm"):
    """SLA forward on the GPU (sla1_forward): O = O_s + O_l proj_o.

    proj_o: float32 [d, d] or [H, d, d], indexed [in, out]. The router matrices
    are optional (None: the block means of Q and K are compared directly).
    Returns (O, mask) or, with debug, (O, mask, debug dict) whose "o_l" is
    Proj(O_l).
    """
    if proj_o is None:
        raise ValueError("proj_o is required")
    return _run(q, k, v, proj_q, proj_k, None, proj_o, kh, kl, mask_in, False, out, mask_out,
                workspace, debug, phi, linear)


def soft_topk(logits: torch.Tensor, k: float, tau: float, *, out: Optional[torch.Tensor] = None,
              lam: Optional[torch.Tensor] = None):
    """SoftTop-k on the GPU (sla_soft_topk): for every row of the float64 device
    tensor `logits` [..., C], Pc = softmax(row) and M = sigmoid((Pc - lambda) / tau)
    with lambda such that the row sums to k. Returns (M float32 [..., C],
    lambda float32 [...])."""
    lib = load_library()
    if logits.dtype != torch.float64 or not logits.is_cuda or logits.dim() < 1:
        raise ValueError("logits must be a float64 device tensor")
    logits = logits.contiguous()
    C = logits.shape[-1]
    rows = logits.numel() // C if C else 0
    if out is None:
        out = torch.empty(logits.shape, dtype=torch.float32, device=logits.device)
    if lam is None:
        lam = torch.empty(logits.shape[:-1], dtype=torch.float32, device=logits.device)
    with torch.cuda.device(logits.device):
        stream = ctypes.c_void_p(torch.cuda.current_stream(logits.device).cuda_stream)
        rc = lib.sla_soft_topk(_ptr(logits), rows, C, float(k), float(tau), _ptr(out), _ptr(lam), stream)
    _check(rc)
    return out, lam


def _backward(q, k, v, alpha, proj_o, mask, dO, workspace, phi, linear="gemm", saved=False):
    lib = load_library()
    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape or dO.shape != q.shape:
        raise ValueError("q, k, v and dO must share one [B, H, N, d] shape")
    if q.dtype not in (torch.bfloat16, torch.float32) or any(t.dtype != q.dtype for t in (k, v, dO)):
        raise ValueError("q, k, v and dO must all be bfloat16 or all float32")
    B, H, N, d = q.shape
    Nb = (N + 63) // 64
    if mask.dtype != torch.int8 or tuple(mask.shape) != (B, H, Nb, Nb):
        raise ValueError("mask must be int8 [B, H, Nb, Nb]")
    hs = 0
    if proj_o is None:
        if alpha is None or alpha.dtype != torch.float32 or alpha.numel() != H:
            raise ValueError("alpha must be float32 with H entries")
    else:
        _check_router("proj_o", proj_o, H, d)
        hs = d * d if proj_o.dim() == 3 else 0
    if not q.is_cuda:
        raise ValueError("q, k, v and dO must be device tensors")
    for name, t in (("k", k), ("v", v), ("alpha", alpha), ("proj_o", proj_o), ("mask", mask), ("dO", dO),
                    ("workspace", workspace)):
        _same_device(name, t, q.device)
    q, k, v, dO, mask = (t.contiguous() for t in (q, k, v, dO, mask))
    alpha = None if alpha is None else alpha.contiguous()
    proj_o = None if proj_o is None else proj_o.contiguous()
    p = make_problem(B, H, N, d, "bf16" if q.dtype == torch.bfloat16 else "f32", 0.0, 0.0,
                     proj_head_stride=hs, phi=phi, linear=linear)
    n = ctypes.c_size_t()
    size_fn = lib.sla_backward_workspace_bytes if proj_o is None else lib.sla1_backward_workspace_bytes
    _check(size_fn(ctypes.byref(p), ctypes.byref(n)))
    if saved:
        if workspace is None or not workspace.is_contiguous():
            raise ValueError("the backward from saved state needs the workspace its forward_train filled")
    elif workspace is None or workspace.numel() * workspace.element_size() < n.value:
        workspace = torch.empty(max(n.value, 256), dtype=torch.uint8, device=q.device)
    dQ = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    dK = torch.empty_like(dQ)
    dV = torch.empty_like(dQ)
    if proj_o is None:
        dpar = torch.empty(H, dtype=torch.float32, device=q.device)
    else:
        dpar = torch.empty(proj_o.shape, dtype=torch.float32, device=q.device)
    with torch.cuda.device(q.device):
        stream = ctypes.c_void_p(torch.cuda.current_stream(q.device).cuda_stream)
        if saved:
            fn = lib.sla_backward_saved if proj_o is None else lib.sla1_backward_saved
        else:
            fn = lib.sla_backward if proj_o is None else lib.sla1_backward
        rc = fn(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha if proj_o is None else proj_o), _ptr(mask),
                _ptr(dO), _ptr(dQ), _ptr(dK), _ptr(dV), _ptr(dpar), _ptr(workspace),
                ctypes.c_size_t(workspace.numel() * workspace.element_size()), stream)
    _check(rc)
    return dQ, dK, dV, dpar


def backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, alpha: torch.Tensor,
             mask: torch.Tensor, dO: torch.Tensor, *, workspace: Optional[torch.Tensor] = None,
             phi: str = "softmax", linear: str = "gemm"):
    """SLA2 backward on the GPU (sla_backward) for the block mask the forward
    pass used: returns (dQ, dK, dV float32 [B, H, N, d], dalpha float32 [H])."""
    return _backward(q, k, v, alpha, None, mask, dO, workspace, phi, linear)


def backward_sla1(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, proj_o: torch.Tensor,
                  mask: torch.Tensor, dO: torch.Tensor, *, workspace: Optional[torch.Tensor] = None,
                  phi: str = "softmax", linear: str = "gemm"):
    """Backward of the SLA formulation O = O_s + O_l proj_o on the GPU
    (sla1_backward): returns (dQ, dK, dV float32 [B, H, N, d], dproj_o float32
    of proj_o's shape)."""
    if proj_o is None:
        raise ValueError("proj_o is required")
    return _backward(q, k, v, None, proj_o, mask, dO, workspace, phi, linear)


def backward_saved(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, alpha: torch.Tensor,
                   mask: torch.Tensor, dO: torch.Tensor, workspace: torch.Tensor, *,
                   phi: str = "softmax", linear: str = "gemm"):
    """SLA2 backward from the state forward_train left in `workspace`
    (sla_backward_saved): the same results as backward(), without running the
    forward again. q, k, v, alpha, mask, phi and linear must be those of the
    forward_train call, and the workspace untouched since."""
    return _backward(q, k, v, alpha, None, mask, dO, workspace, phi, linear, saved=True)


def backward_sla1_saved(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, proj_o: torch.Tensor,
                        mask: torch.Tensor, dO: torch.Tensor, workspace: torch.Tensor, *,
                        phi: str = "softmax", linear: str = "gemm"):
    """SLA backward from the state forward_sla1_train left in `workspace`
    (sla1_backward_saved)."""
    if proj_o is None:
        raise ValueError("proj_o is required")
    return _backward(q, k, v, None, proj_o, mask, dO, workspace, phi, linear, saved=True)


class Plan:
    """A prepared sla_forward (or, with proj_o, sla1_forward) call: the problem, the device buffers and the
    ctypes argument list are built once, so repeated calls only enqueue work
    (used by the benchmark and by callers that run the same shape often)."""

    def __init__(self, q, k, v, proj_q, proj_k, alpha, kh, kl, mask_in=None, quant=False,
                 phi="softmax", proj_o=None, linear="gemm"):
        lib = load_library()
        hs = validate_forward_args(q, k, v, proj_q, proj_k, alpha, proj_o, mask_in)
        for name, t in (("proj_q", proj_q), ("proj_k", proj_k), ("alpha", alpha), ("proj_o", proj_o),
                        ("mask_in", mask_in)):
            if t is not None and not t.is_contiguous():
                raise ValueError(f"{name} must be contiguous (a Plan keeps raw pointers to it)")
        B, H, N, d = q.shape
        Nb = (N + 63) // 64
        dev = q.device
        self.problem = make_problem(B, H, N, d, "bf16" if q.dtype == torch.bfloat16 else "f32",
                                    kh, kl, quant, hs, phi, linear)
        self.sla1 = proj_o is not None
        self.nbytes = workspace_bytes(self.problem)
        self.workspace = torch.empty(max(self.nbytes, 256), dtype=torch.uint8, device=dev)
        self.out = torch.empty_like(q)
        self.mask = None if mask_in is not None else torch.empty((B, H, Nb, Nb), dtype=torch.int8,
                                                                 device=dev)
        self._keep = (q, k, v, proj_q, proj_k, alpha, mask_in, proj_o)
        self.device = dev
        self.lib = lib
        self._args = [ctypes.byref(self.problem), _ptr(q), _ptr(k), _ptr(v), _ptr(proj_q),
                      _ptr(proj_k), _ptr(proj_o if self.sla1 else alpha), _ptr(mask_in),
                      _ptr(self.out), _ptr(self.mask), _ptr(self.workspace),
                      ctypes.c_size_t(self.nbytes)]
        self._fwd = lib.sla1_forward if self.sla1 else lib.sla_forward
        self._fwd_debug = lib.sla1_forward_debug if self.sla1 else lib.sla_forward_debug
        self.dims = (B, H, N, d, Nb)

    def run(self, events=None):
        """Enqueues one forward pass on torch's current stream. `events`: optional
        sequence of 6 raw hipEvent_t handles recorded around the five kernels."""
        stream = ctypes.c_void_p(torch.cuda.current_stream(self.device).cuda_stream)
        if events is None:
            rc = self._fwd(*self._args, stream)
        else:
            dbg = Debug(None, None, None, None, None, (ctypes.c_void_p * 6)(*events))
            rc = self._fwd_debug(*self._args, stream, ctypes.byref(dbg))
        _check(rc)
        return self.out


# hipEventDisableSystemFence: the event's record skips the system-scope release
# (an L2 writeback and invalidation), which would otherwise stall the stream for
# several microseconds between the kernels it brackets and make the following
# kernel start on a cold L2. Timestamps stay valid once the device has been
# synchronised.
HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000


class HipEvents:
    """Raw HIP events through the HIP runtime (for per-kernel timing), created
    without a system-scope fence so that recording them does not perturb the
    kernels they bracket."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if self.hip.hipEventCreateWithFlags(ctypes.byref(e), HIP_EVENT_DISABLE_SYSTEM_FENCE) != 0:
                raise RuntimeError("hipEventCreateWithFlags failed")
            out.append(e.value)
        return out

    def record(self, ev, stream) -> None:
        """Records raw event ev on the raw hipStream_t stream (an int or None)."""
        if self.hip.hipEventRecord(ctypes.c_void_p(ev), ctypes.c_void_p(stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, evs):
        for e in evs:
            self.hip.hipEventDestroy(ctypes.c_void_p(e))
