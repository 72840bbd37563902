"""Seeded synthetic Q, K, V, router and alpha tensors for the SLA workloads.

Recipe (the pages use activations of Wan2.1 video DiTs, which are not available;
these inputs stand in for them with the same shapes and a calibrated structure):

* tokens are laid out in raster order n = (t*Hg + y)*Wg + x over the latent grid;
* p_n is a 3-axis sin/cos position embedding: the d channels are split into
  (d - 4*(d//6), 2*(d//6), 2*(d//6)) for (t, y, x); an axis with m channels uses the
  frequencies w_k = 10000^(-2k/m), k < m/2, and emits sin(pos*w_k) then
  cos(pos*w_k), so |p_n|^2 = d/2;
* q_n = A_q p_n + 0.5*eps and k_n = A_k p_n + 0.5*eps' with independent
  A_q, A_k of i.i.d. N(0, s^2/d) entries per (batch, head); V ~ N(0, 1);
* s = 3.4 makes dense softmax attention as peaked as the pages report for
  Wan2.1 (SLA paper summary, Fig. 1: about 8.1% of the weights exceed 1/N and
  about 45% lie below 1/(100N)); a CPU test measures both fractions;
* the learned router is proj = I + 0.1*N(0, 1/d) (one [d, d] matrix shared by
  all heads), alpha is per head, constant or uniform.

Every draw comes from its own counter-keyed stream
SeedSequence([seed, stream, b, h]), so any (b, h) slice can be regenerated alone.
Values are drawn in float64 and rounded once to the workload dtype (float32, or
float32 then bfloat16 with round-to-nearest-even); both the oracle and the HIP
path read exactly these rounded values.
"""

from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from .configs import WorkloadConfig

POSEMB_SCALE = 3.4

# stream ids of the counter-keyed generators
_S_AQ, _S_AK, _S_NQ, _S_NK, _S_V, _S_PQ, _S_PK, _S_ALPHA, _S_Q, _S_K, _S_PO = range(11)


def _rng(seed: int, stream: int, b: int = 0, h: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, stream, b, h]))


def sincos_posemb(grid, d: int, N: Optional[int] = None) -> np.ndarray:
    """[N, d] float64 3-axis sin/cos embedding of a (t, h, w) grid in raster order."""
    T, Hg, Wg = grid
    dh = 2 * (d // 6)
    dw = 2 * (d // 6)
    dt = d - dh - dw
    n = np.arange(T * Hg * Wg if N is None else N)
    t = n // (Hg * Wg)
    y = (n // Wg) % Hg
    x = n % Wg
    cols = []
    for pos, m in ((t, dt), (y, dh), (x, dw)):
        k = np.arange(m // 2)
        w = 10000.0 ** (-2.0 * k / m)
        ang = pos[:, None].astype(np.float64) * w[None, :]
        cols.append(np.sin(ang))
        cols.append(np.cos(ang))
    return np.concatenate(cols, axis=1)


@dataclass
class Inputs:
    cfg: WorkloadConfig
    B: int
    H: int
    N: int
    d: int
    q: torch.Tensor        # [B, H, N, d] float32 or bfloat16, CPU
    k: torch.Tensor
    v: torch.Tensor
    proj_q: torch.Tensor   # [d, d] float32
    proj_k: torch.Tensor
    alpha: torch.Tensor    # [H] float32
    kh: float
    kl: float

    @property
    def torch_dtype(self):
        return self.q.dtype


def _to_dtype(x: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t if dtype == "f32" else t.to(torch.bfloat16)


def make_inputs(cfg: WorkloadConfig, *, B: Optional[int] = None, H: Optional[int] = None,
                N: Optional[int] = None, kh: Optional[float] = None,
                kl: Optional[float] = None) -> Inputs:
    """Build the seeded inputs of `cfg`, optionally with a smaller B, H or N.

    A smaller N keeps the first N tokens of the raster order; a smaller B or H
    keeps the leading slices, which are bit-identical to those of the full size.
    """
    B = cfg.B if B is None else B
    H = cfg.H if H is None else H
    N = cfg.N if N is None else N
    d = cfg.d
    tdt = torch.float32 if cfg.dtype == "f32" else torch.bfloat16
    q = torch.empty((B, H, N, d), dtype=tdt)
    k = torch.empty((B, H, N, d), dtype=tdt)
    v = torch.empty((B, H, N, d), dtype=tdt)
    P = sincos_posemb(cfg.grid, d, N) if cfg.qk == "posemb" else None
    sa = POSEMB_SCALE / np.sqrt(d)
    for b in range(B):
        for h in range(H):
            if cfg.qk == "posemb":
                Aq = _rng(cfg.seed, _S_AQ, b, h).standard_normal((d, d)) * sa
                Ak = _rng(cfg.seed, _S_AK, b, h).standard_normal((d, d)) * sa
                qn = P @ Aq.T + 0.5 * _rng(cfg.seed, _S_NQ, b, h).standard_normal((N, d))
                kn = P @ Ak.T + 0.5 * _rng(cfg.seed, _S_NK, b, h).standard_normal((N, d))
            else:
                qn = _rng(cfg.seed, _S_Q, b, h).standard_normal((N, d))
                kn = _rng(cfg.seed, _S_K, b, h).standard_normal((N, d))
            vn = _rng(cfg.seed, _S_V, b, h).standard_normal((N, d))
            q[b, h] = _to_dtype(qn, cfg.dtype)
            k[b, h] = _to_dtype(kn, cfg.dtype)
            v[b, h] = _to_dtype(vn, cfg.dtype)
    if cfg.router == "identity":
        pq = np.eye(d)
        pk = np.eye(d)
    else:
        pq = np.eye(d) + 0.1 * _rng(cfg.seed, _S_PQ).standard_normal((d, d)) / np.sqrt(d)
        pk = np.eye(d) + 0.1 * _rng(cfg.seed, _S_PK).standard_normal((d, d)) / np.sqrt(d)
    if cfg.alpha[0] == "const":
        al = np.full(cfg.H, cfg.alpha[1])
    else:
        al = _rng(cfg.seed, _S_ALPHA).uniform(cfg.alpha[1], cfg.alpha[2], size=cfg.H)
    return Inputs(cfg, B, H, N, d, q, k, v,
                  torch.from_numpy(pq.astype(np.float32)),
                  torch.from_numpy(pk.astype(np.float32)),
                  torch.from_numpy(al[:H].astype(np.float32)),
                  cfg.kh if kh is None else kh, cfg.kl if kl is None else kl)


def make_proj_o(cfg: WorkloadConfig, *, H: Optional[int] = None, per_head: bool = False) -> torch.Tensor:
    """SLA's learned output map Proj (O = O_s + Proj(O_l)) as float32, indexed
    [in, out]: one [d, d] matrix, or [H, d, d] with per_head. Entries are
    i.i.d. N(0, 1/d), a map of unit gain (the pages give no initialisation);
    head h of the per-head form has its own stream, so the leading heads match
    at any H."""
    d = cfg.d
    if not per_head:
        w = _rng(cfg.seed, _S_PO).standard_normal((d, d)) / np.sqrt(d)
    else:
        H = cfg.H if H is None else H
        w = np.stack([_rng(cfg.seed, _S_PO, 0, h + 1).standard_normal((d, d)) / np.sqrt(d)
                      for h in range(H)])
    return torch.from_numpy(w.astype(np.float32))
