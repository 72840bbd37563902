"""The float64 oracle's outputs for many query blocks of one head, spread over
worker processes (test infrastructure; no test functions here).

Workers are started with the "spawn" method and import only numpy and the
oracle, so that nothing of a GPU runtime the parent holds is inherited; each
gets the head's inputs once and a share of the query blocks, with two BLAS
threads of its own.
"""

import multiprocessing as mp
import os

import numpy as np

_HEAD = {}


def _init(q, k, v, proj_q, proj_k, alpha, mask, kh, kl, feature, proj_o):
    from threadpoolctl import threadpool_limits
    threadpool_limits(2)
    _HEAD.update(q=q, k=k, v=v, proj_q=proj_q, proj_k=proj_k, alpha=alpha, mask=mask, kh=kh, kl=kl,
                 feature=feature, proj_o=proj_o)


def _run(blocks):
    import oracle as orc
    h = _HEAD
    r = orc.forward(h["q"], h["k"], h["v"], h["proj_q"], h["proj_k"], h["alpha"], h["kh"], h["kl"],
                    mask_in=h["mask"], query_blocks={(0, 0): blocks}, feature=h["feature"], proj_o=h["proj_o"])
    return blocks, r.O[(0, 0)], r.O_s[(0, 0)], r.O_l[(0, 0)]


def head_outputs(x, b, h, mask, blocks=None, feature="softmax", proj_o=None, router=True, workers=None):
    """(O, O_s, O_l) [len(rows), d] float64 of head (b, h) of the seeded inputs
    x (workloads.Inputs) for the given query blocks (default all), in block
    order, with the block mask `mask` [B, H, Nb, Nb] injected."""
    N = x.N
    Nb = (N + 63) // 64
    blocks = list(range(Nb)) if blocks is None else sorted(blocks)
    workers = workers or max(1, min(8, len(os.sched_getaffinity(0)) // 2))
    f64 = lambda t: t[b:b + 1, h:h + 1].double().numpy()
    alpha = None if proj_o is not None else x.alpha[h:h + 1].double().numpy()
    po = None
    if proj_o is not None:
        po = proj_o.double().numpy()
        po = po[h] if po.ndim == 3 else po
    pq = pk = None
    if router and proj_o is None:
        pq, pk = x.proj_q.double().numpy(), x.proj_k.double().numpy()
        if pq.ndim == 3:
            pq, pk = pq[h], pk[h]
    m = np.ascontiguousarray(mask[b:b + 1, h:h + 1])
    chunks = [blocks[i::workers * 4] for i in range(workers * 4)]
    chunks = [c for c in chunks if c]
    ctx = mp.get_context("spawn")
    with ctx.Pool(workers, initializer=_init,
                  initargs=(f64(x.q), f64(x.k), f64(x.v), pq, pk, alpha, m, x.kh, x.kl, feature, po)) as pool:
        parts = pool.map(_run, chunks)
    rows = {}
    for blks, O, Os, Ol in parts:
        off = 0
        for i in blks:
            n = min(64, N - 64 * i)
            rows[i] = (O[off:off + n], Os[off:off + n], Ol[off:off + n])
            off += n
    cat = lambda k: np.concatenate([rows[i][k] for i in blocks], axis=0)
    return cat(0), cat(1), cat(2)
