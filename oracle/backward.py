"""Float64 CPU oracle of the SLA2 backward pass (gradients for a fixed mask).

TEST INFRASTRUCTURE ONLY, like the rest of this package: imported by the tests
and by the benchmark's cpu_baseline leg, never by the product path; it shares
no code with the HIP path.

The pages describe the backward only in outline (SLA explainer, section 2.3:
the FlashAttention backward restricted to the blocks with Mc = 1 for the
sparse path, the chain rule through phi(Q), phi(K) and V with per-block
accumulation for the linear path; SLA paper summary, Fig. 6's backward-kernel
speed). They print no formulas for it, so the oracle is the definition: the
explicit forward of sla_oracle.forward (masked softmax over the critical
tokens, explicit phi(Q) phi(K)^T restricted to marginal tokens and
row-normalised, the alpha mix), written with torch float64 operations on the
CPU and differentiated by autograd. The mask is an input (it is a hard,
piecewise-constant function of Q and K, so no gradient flows through the
router, the pooling or the ranking).

The SLA formulation (SLA paper summary, section 4, step 4 and its
final-output formula) fuses the branches as O = O_s + O_l W with a learned
d x d map W indexed [in, out] (one shared matrix or one per head); with
proj_o given, the same explicit forward uses that fusion and the gradients
include dW (summed over the batch, and over the heads when W is shared). Both
formulations take phi = softmax over the features or elu + 1 elementwise
(SLA paper summary, Eq. 3's symbols and Table 2).
"""

from typing import Dict, Tuple

import numpy as np
import torch

BLOCK = 64


def _token_masks(mask_row: np.ndarray, N: int) -> Tuple[torch.Tensor, torch.Tensor]:
    m = torch.from_numpy(np.repeat(np.asarray(mask_row), BLOCK)[:N])
    return m == 1, m == 0


def forward_torch(Q, K, V, alpha, mask, phi: str = "softmax", proj_o=None):
    """Explicit forward in torch float64 for a fixed block mask [B, H, Nb, Nb];
    Q, K, V [B, H, N, d] float64 tensors (requires_grad as wanted), alpha [H]
    (SLA2 mix) or, with proj_o ([d, d] or [H, d, d]), the SLA fusion
    O = O_s + O_l proj_o (alpha unused). Returns (O, O_s, O_l)."""
    B, H, N, d = Q.shape
    Nb = (N + BLOCK - 1) // BLOCK
    outs, outs_s, outs_l = [], [], []
    for b in range(B):
        ob, osb, olb = [], [], []
        for h in range(H):
            q, k, v = Q[b, h], K[b, h], V[b, h]
            S = (q @ k.T) / np.sqrt(d)
            if phi == "softmax":
                fq, fk = torch.softmax(q, dim=-1), torch.softmax(k, dim=-1)
            else:
                fq, fk = torch.nn.functional.elu(q) + 1.0, torch.nn.functional.elu(k) + 1.0
            A = fq @ fk.T
            rows_s, rows_l = [], []
            for i in range(Nb):
                t0, t1 = i * BLOCK, min((i + 1) * BLOCK, N)
                crit, marg = _token_masks(mask[b, h, i], N)
                if crit.any():
                    Si = S[t0:t1].masked_fill(~crit[None, :], float("-inf"))
                    rows_s.append(torch.softmax(Si, dim=-1) @ v)
                else:
                    rows_s.append(torch.zeros(t1 - t0, d, dtype=Q.dtype))
                if marg.any():
                    Ai = A[t0:t1] * marg[None, :].to(Q.dtype)
                    rows_l.append((Ai @ v) / Ai.sum(dim=-1, keepdim=True))
                else:
                    rows_l.append(torch.zeros(t1 - t0, d, dtype=Q.dtype))
            Os, Ol = torch.cat(rows_s), torch.cat(rows_l)
            osb.append(Os)
            olb.append(Ol)
            if proj_o is None:
                ob.append(alpha[h] * Os + (1.0 - alpha[h]) * Ol)
            else:
                ob.append(Os + Ol @ (proj_o[h] if proj_o.dim() == 3 else proj_o))
        outs.append(torch.stack(ob))
        outs_s.append(torch.stack(osb))
        outs_l.append(torch.stack(olb))
    return torch.stack(outs), torch.stack(outs_s), torch.stack(outs_l)


def backward(Q, K, V, alpha, mask, dO, phi: str = "softmax", proj_o=None) -> Dict[str, np.ndarray]:
    """Gradients of sum(O * dO) with respect to Q, K, V and alpha (SLA2) or
    proj_o (SLA, when proj_o is given), float64. Inputs are upcast exactly
    (bf16 / f32 -> f64). Returns numpy arrays dQ, dK, dV [B, H, N, d] and
    dalpha [H] (summed over the batch) or dproj_o (proj_o's shape)."""
    f64 = lambda x: (x.detach().to("cpu", torch.float64) if hasattr(x, "detach")
                     else torch.from_numpy(np.asarray(x, dtype=np.float64)))
    q = f64(Q).requires_grad_(True)
    k = f64(K).requires_grad_(True)
    v = f64(V).requires_grad_(True)
    g = f64(dO)
    if proj_o is None:
        a = f64(alpha).reshape(-1).requires_grad_(True)
        w = None
    else:
        a = None
        w = f64(proj_o).requires_grad_(True)
    O, _, _ = forward_torch(q, k, v, a, np.asarray(mask), phi, w)
    (O * g).sum().backward()
    out = {"dQ": q.grad.numpy(), "dK": k.grad.numpy(), "dV": v.grad.numpy()}
    if w is None:
        out["dalpha"] = a.grad.numpy()
    else:
        out["dproj_o"] = w.grad.numpy()
    return out


def dq_rows(Q, K, V, alpha, mask, dO, b: int, h: int, blocks, phi: str = "softmax",
            proj_o=None) -> Dict[int, np.ndarray]:
    """dQ of the given query blocks of head (b, h), float64. The rows of O in
    query block i depend on q only through that block's own rows, so the
    gradient of sum(O_i * dO_i) with respect to them is dQ there; only those
    rows' forward is formed (the same explicit definition as forward_torch)."""
    f64 = lambda x: (x.detach().to("cpu", torch.float64) if hasattr(x, "detach")
                     else torch.from_numpy(np.asarray(x, dtype=np.float64)))
    k, v = f64(K[b, h]), f64(V[b, h])
    if proj_o is None:
        a, wo = float(f64(alpha).reshape(-1)[h]), None
    else:
        wo = f64(proj_o)
        wo = wo[h] if wo.dim() == 3 else wo
    N, d = k.shape
    fk = torch.softmax(k, dim=-1) if phi == "softmax" else torch.nn.functional.elu(k) + 1.0
    out = {}
    for i in blocks:
        t0, t1 = i * BLOCK, min((i + 1) * BLOCK, N)
        qi = f64(Q[b, h, t0:t1]).requires_grad_(True)
        gi = f64(dO[b, h, t0:t1])
        crit, marg = _token_masks(np.asarray(mask)[b, h, i], N)
        O = torch.zeros(t1 - t0, d, dtype=torch.float64)
        if crit.any():
            S = ((qi @ k.T) / np.sqrt(d)).masked_fill(~crit[None, :], float("-inf"))
            Os = torch.softmax(S, dim=-1) @ v
            O = O + (Os if wo is not None else a * Os)
        if marg.any():
            fq = torch.softmax(qi, dim=-1) if phi == "softmax" else torch.nn.functional.elu(qi) + 1.0
            A = (fq @ fk.T) * marg[None, :].to(torch.float64)
            Ol = (A @ v) / A.sum(dim=-1, keepdim=True)
            O = O + (Ol @ wo if wo is not None else (1.0 - a) * Ol)
        (O * gi).sum().backward()
        out[int(i)] = qi.grad.numpy()
    return out
