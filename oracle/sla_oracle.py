"""Float64 CPU oracle of the SLA / SLA2 sparse-linear attention forward pass.

TEST INFRASTRUCTURE ONLY. It is imported by the tests, by the smoke check of the
package entry module and by the cpu_baseline leg of the benchmark; the product
path (the HIP library and its Python binding) never imports, calls or links it.
It shares no code, table or helper with the HIP path.

What it computes, in the order the pages give (citations name the page and the
section / equation on it):

1. 64-token blocks of queries and keys (SLA explainer, section 2.2 item 1;
   SLA paper summary, section 4, symbols of Eq. 3).
2. Router: Q~ = Q proj_q, K~ = K proj_k, two learned projection matrices
   (SLA2 article, the "learned router" paragraph; SLA2 cross-paper synthesis,
   section 5.2). Then mean pooling along the sequence inside each block
   (SLA paper summary, section 4 step 1 and Eq. 1).
3. Compressed attention Pc = softmax(pool(Q) pool(K)^T / sqrt(d)) (Eq. 1).
4. Classification Mc[i, j] = 1 for the top kh% of row i, -1 for the bottom
   kl%, 0 otherwise (Eq. 2).
5. Sparse branch: softmax attention restricted to the critical blocks
   (section 4 step 3, first bullet), written out as an explicit masked softmax.
6. Linear branch on the marginal blocks, phi = softmax over the features
   (Eq. 3; feature-map choice: SLA explainer section 3.2, SLA paper summary
   Table 2), written out as the explicit matrix phi(Q) phi(K)^T restricted to
   marginal entries and row-normalised.
7. Negligible blocks are skipped (section 4 step 3, third bullet).
8. SLA2 mix O = alpha * O_s + (1 - alpha) * O_l (SLA2 article, the
   "learnable mixing ratio" paragraph).

The SLA (v1) formulation differs in two places, both selectable here:
* output fusion O = O_s + Proj(O_l) with a learned d x d linear map Proj
  (SLA paper summary, section 4, step 4 and the final-output formula; SLA
  explainer, section 2.1 on Eq. 6's projection), read as O_l @ proj_o with
  proj_o indexed [in, out] like the router matrices, no bias;
* the feature map phi(x) = elu(x) + 1, elementwise (SLA paper summary, the
  symbols of Eq. 3 and Table 2's "SLA (elu+1)" row; SLA2 blog, section 4.2),
  besides the softmax (SLA explainer, section 3.2).
SLA (v1) has no learned router: its compressed map pools Q and K directly,
which is proj_q = proj_k = None here (the identity).

Readings where the pages are silent (all listed in the design notes):
counts n_h = max(1, floor(kh*Nb + 1e-9)) when kh > 0, n_l = floor(kl*Nb + 1e-9);
one total order per row, logit descending then block index ascending, critical
taken from its head and negligible from its tail; proj indexed [in, out]; the
ragged last block pools over its valid tokens only; phi acts on the
un-projected Q and K; an empty critical (or marginal) set gives a zero sparse
(or linear) output; alpha is one float per head.

Parity status: every function here is pinned by CPU tests against closed forms,
library routines on special cases (dense softmax attention at kh = 100%, pure
linear attention at kh = kl = 0), invariances and an independent scalar
brute force on tiny inputs.
"""

from dataclasses import dataclass, field
from typing import Dict, Iterable, Optional, Tuple

import numpy as np

BLOCK = 64


def num_blocks(N: int) -> int:
    """Number of 64-token blocks covering N tokens; the last may be ragged."""
    return (N + BLOCK - 1) // BLOCK


def block_counts(Nb: int, kh: float, kl: float) -> Tuple[int, int]:
    """Critical and negligible block counts per query-block row (Eq. 2's top
    kh% / bottom kl%). The pages give percentages only; the count is the floor
    of kh*Nb (a small epsilon absorbs products such as 0.29*100 = 28.999...),
    at least one critical block whenever kh > 0."""
    if not (0.0 <= kh <= 1.0 and 0.0 <= kl <= 1.0):
        raise ValueError("kh and kl must lie in [0, 1]")
    n_h = 0 if kh <= 0.0 else max(1, int(np.floor(kh * Nb + 1e-9)))
    n_h = min(n_h, Nb)
    n_l = int(np.floor(kl * Nb + 1e-9))
    if n_h + n_l > Nb:
        raise ValueError("kh and kl select more blocks than a row has")
    return n_h, n_l


def phi(x: np.ndarray) -> np.ndarray:
    """Feature map: softmax over the last (feature) axis, float64."""
    z = x - x.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=-1, keepdims=True)


def phi_elu1(x: np.ndarray) -> np.ndarray:
    """Feature map ELU+1, elementwise: x + 1 where x > 0, exp(x) elsewhere
    (ELU with unit scale, shifted by one so that every feature is positive)."""
    return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))


FEATURE_MAPS = {"softmax": phi, "elu1": phi_elu1}


def router_pool(X: np.ndarray, proj: np.ndarray) -> np.ndarray:
    """Project every token with the router matrix ([in, out]), then take the
    mean of each 64-token block over its valid tokens. X: [N, d] -> [Nb, d]."""
    N = X.shape[0]
    Xp = X @ proj
    Nb = num_blocks(N)
    out = np.empty((Nb, Xp.shape[1]), dtype=np.float64)
    for i in range(Nb):
        out[i] = Xp[i * BLOCK:min((i + 1) * BLOCK, N)].mean(axis=0)
    return out


def compressed_scores(qbar: np.ndarray, kbar: np.ndarray, d: int):
    """Eq. 1: logits s = pool(Q) pool(K)^T / sqrt(d) and Pc = row softmax(s)."""
    s = (qbar @ kbar.T) / np.sqrt(d)
    z = s - s.max(axis=1, keepdims=True)
    e = np.exp(z)
    return s, e / e.sum(axis=1, keepdims=True)


def classify(s: np.ndarray, n_h: int, n_l: int) -> np.ndarray:
    """Eq. 2 with one total order per row: larger logit first, lower block index
    first among equal logits. Head n_h -> 1 (critical), tail n_l -> -1
    (negligible), the rest 0 (marginal). Ranking the logits ranks Pc identically."""
    Nq, Nk = s.shape
    mask = np.zeros((Nq, Nk), dtype=np.int8)
    cols = np.arange(Nk)
    for i in range(Nq):
        order = np.lexsort((cols, -s[i]))  # primary key -s (ascending), then index
        mask[i, order[:n_h]] = 1
        if n_l > 0:
            mask[i, order[Nk - n_l:]] = -1
    return mask


def token_mask(mask_row: np.ndarray, value: int, N: int) -> np.ndarray:
    """Expand one block-mask row to a boolean over the N key tokens."""
    return np.repeat(mask_row == value, BLOCK)[:N]


def sparse_branch(q: np.ndarray, K: np.ndarray, V: np.ndarray, crit: np.ndarray) -> np.ndarray:
    """Softmax attention of the query rows q over the critical key tokens only,
    as an explicit masked softmax over all N keys. Zero if no key is critical."""
    d = q.shape[1]
    if not crit.any():
        return np.zeros((q.shape[0], V.shape[1]))
    S = (q @ K.T) / np.sqrt(d)
    S = np.where(crit[None, :], S, -np.inf)
    S = S - S.max(axis=1, keepdims=True)
    P = np.exp(S)
    return (P @ V) / P.sum(axis=1, keepdims=True)


def linear_branch(q: np.ndarray, K: np.ndarray, V: np.ndarray, marg: np.ndarray,
                  feature: str = "softmax") -> np.ndarray:
    """Linear attention of the query rows over the marginal key tokens:
    A = phi(q) phi(K)^T kept on marginal entries, O_l = A V / rowsum(A).
    Zero if no key is marginal. feature: "softmax" or "elu1"."""
    f = FEATURE_MAPS[feature]
    if not marg.any():
        return np.zeros((q.shape[0], V.shape[1]))
    A = f(q) @ f(K).T
    A = np.where(marg[None, :], A, 0.0)
    return (A @ V) / A.sum(axis=1, keepdims=True)


@dataclass
class OracleResult:
    n_h: int
    n_l: int
    mask: np.ndarray                 # [B, H, Nb, Nb] int8
    O: Dict[Tuple[int, int], np.ndarray] = field(default_factory=dict)     # (b,h) -> [N,d] or rows
    O_s: Dict[Tuple[int, int], np.ndarray] = field(default_factory=dict)
    O_l: Dict[Tuple[int, int], np.ndarray] = field(default_factory=dict)
    O_lp: Dict[Tuple[int, int], np.ndarray] = field(default_factory=dict)  # Proj(O_l), SLA fusion
    pooled_q: Optional[np.ndarray] = None   # [B, H, Nb, d]
    pooled_k: Optional[np.ndarray] = None
    logits: Optional[np.ndarray] = None     # [B, H, Nb, Nb]
    Pc: Optional[np.ndarray] = None
    rows: Dict[Tuple[int, int], np.ndarray] = field(default_factory=dict)  # (b,h) -> query blocks


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):  # torch tensor: upcast exactly (bf16/f32 -> f64)
        import torch
        return x.detach().to(device="cpu", dtype=torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def forward(Q, K, V, proj_q, proj_k, alpha, kh: float, kl: float,
            mask_in=None, query_blocks: Optional[Dict[Tuple[int, int], Iterable[int]]] = None,
            heads: Optional[Iterable[Tuple[int, int]]] = None,
            compute_outputs: bool = True, feature: str = "softmax",
            proj_o=None) -> OracleResult:
    """SLA2 (or, with proj_o, SLA) forward pass in float64.

    Q, K, V: [B, H, N, d] (numpy or torch, any float dtype; upcast exactly).
    proj_q, proj_k: [d, d] shared by all heads, or [H, d, d]; both None for
    no router projection (the block means of Q and K themselves).
    alpha: [H] (SLA2 mix; ignored with proj_o).  mask_in: optional
    [B, H, Nb, Nb] block mask in {1, 0, -1} that replaces steps 2-4.
    feature: the linear branch's feature map, "softmax" or "elu1".
    proj_o: None for the SLA2 mix, else the SLA output map ([d, d] or
    [H, d, d], indexed [in, out]): O = O_s + O_l @ proj_o.
    heads: the (b, h) pairs to process (default all).
    query_blocks: optional per-(b, h) subset of query blocks for which O is
    produced (the mask is always formed for every row of a processed head).
    Outputs per (b, h) are [len(rows)*64 (clipped), d] arrays of the selected
    query blocks' tokens, in block order.
    """
    Q = _f64(Q)
    K = _f64(K)
    V = _f64(V)
    B, H, N, d = Q.shape
    if (proj_q is None) != (proj_k is None):
        raise ValueError("proj_q and proj_k are both given or both None")
    pq = np.eye(d) if proj_q is None else _f64(proj_q)
    pk = np.eye(d) if proj_k is None else _f64(proj_k)
    if feature not in FEATURE_MAPS:
        raise ValueError("unknown feature map %r" % (feature,))
    po = None if proj_o is None else _f64(proj_o)
    al = None if po is not None else _f64(alpha).reshape(-1)
    Nb = num_blocks(N)
    n_h, n_l = block_counts(Nb, kh, kl)
    res = OracleResult(n_h, n_l, np.zeros((B, H, Nb, Nb), dtype=np.int8))
    if mask_in is None:
        res.pooled_q = np.zeros((B, H, Nb, d))
        res.pooled_k = np.zeros((B, H, Nb, d))
        res.logits = np.zeros((B, H, Nb, Nb))
        res.Pc = np.zeros((B, H, Nb, Nb))
    hs = [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)
    for (b, h) in hs:
        if mask_in is None:
            pqh = pq[h] if pq.ndim == 3 else pq
            pkh = pk[h] if pk.ndim == 3 else pk
            qbar = router_pool(Q[b, h], pqh)
            kbar = router_pool(K[b, h], pkh)
            s, Pc = compressed_scores(qbar, kbar, d)
            m = classify(s, n_h, n_l)
            res.pooled_q[b, h], res.pooled_k[b, h] = qbar, kbar
            res.logits[b, h], res.Pc[b, h] = s, Pc
        else:
            m = np.asarray(mask_in[b, h], dtype=np.int8)
        res.mask[b, h] = m
        if not compute_outputs:
            continue
        rows = list(range(Nb)) if query_blocks is None else sorted(query_blocks.get((b, h), []))
        res.rows[(b, h)] = np.asarray(rows, dtype=np.int64)
        Os, Ol = [], []
        for i in rows:
            t0, t1 = i * BLOCK, min((i + 1) * BLOCK, N)
            q = Q[b, h, t0:t1]
            Os.append(sparse_branch(q, K[b, h], V[b, h], token_mask(m[i], 1, N)))
            Ol.append(linear_branch(q, K[b, h], V[b, h], token_mask(m[i], 0, N), feature))
        Os = np.concatenate(Os, axis=0) if Os else np.zeros((0, d))
        Ol = np.concatenate(Ol, axis=0) if Ol else np.zeros((0, d))
        res.O_s[(b, h)] = Os
        res.O_l[(b, h)] = Ol
        if po is None:
            res.O[(b, h)] = al[h] * Os + (1.0 - al[h]) * Ol
        else:
            poh = po[h] if po.ndim == 3 else po
            res.O_lp[(b, h)] = Ol @ poh
            res.O[(b, h)] = Os + res.O_lp[(b, h)]
    return res


def token_rows(rows: Iterable[int], N: int) -> np.ndarray:
    """Token indices covered by the given query blocks, in block order."""
    out = [np.arange(i * BLOCK, min((i + 1) * BLOCK, N)) for i in rows]
    return np.concatenate(out) if out else np.zeros(0, dtype=np.int64)


def compressed_map(logits: np.ndarray) -> np.ndarray:
    """Pc = row softmax of the compressed logits (Eq. 1), float64."""
    s = np.asarray(logits, dtype=np.float64)
    e = np.exp(s - s.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    # 1 / (1 + e^-x) written so that neither branch overflows
    out = np.empty_like(x)
    pos = x >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-x[pos]))
    ex = np.exp(x[~pos])
    out[~pos] = ex / (1.0 + ex)
    return out


def soft_topk(logits, k: float, tau: float):
    """SoftTop-k of the compressed attention map, the differentiable stand-in
    for Eq. 2's top-k in SLA2's first training stage (SLA2 article, the
    two-stage training paragraphs, stage 1; SLA2 cross-paper synthesis, §3,
    the item on the cost of the binary search for lambda_i).

    For every row i of Pc = softmax(logits): M[i, j] = sigmoid((Pc[i, j] -
    lambda_i) / tau), with lambda_i the value at which the row sums to k,
    found by binary search (the row sum falls strictly from the row length to
    0 as lambda rises). Readings: the sigmoid acts on Pc, the quantity the
    hard top-k ranks; k is a count in [0, row length] (the hard top-k's n_h
    makes tau -> 0 recover that mask); k = 0 gives zeros with lambda = +inf,
    k = row length ones with lambda = -inf.

    logits: [..., C] float64. Returns (M [..., C] float64, lambda [...] float64).
    The search halves a bracket on which the row sum crosses k until its
    midpoint no longer moves in float64.
    """
    if not tau > 0:
        raise ValueError("tau must be positive")
    P = compressed_map(logits)
    C = P.shape[-1]
    if not 0.0 <= k <= C:
        raise ValueError("k must lie in [0, row length]")
    rows = P.reshape(-1, C)
    M = np.empty_like(rows)
    lam = np.empty(rows.shape[0])
    for r in range(rows.shape[0]):
        p = rows[r]
        if k == 0:
            M[r], lam[r] = 0.0, np.inf
            continue
        if k == C:
            M[r], lam[r] = 1.0, -np.inf
            continue
        # at lo every term is above k / C, at hi every term is below k / C
        lo = p.min() - 60.0 * tau
        hi = p.max() + 60.0 * tau
        while True:
            mid = 0.5 * (lo + hi)
            if mid <= lo or mid >= hi:
                break
            if _sigmoid((p - mid) / tau).sum() > k:
                lo = mid
            else:
                hi = mid
        lam[r] = 0.5 * (lo + hi)
        M[r] = _sigmoid((p - lam[r]) / tau)
    return M.reshape(P.shape), lam.reshape(P.shape[:-1])
