"""Benchmark of the SLA2 forward pass on one MI355X.

A step is one full forward pass (pooling, scores + classification, h/z, the
marginal sums, sparse attention + linear branch + mix) over one batch of
seeded synthetic inputs already resident in HBM. The headline workload is the
Wan2.1-1.3B attention shape at 95% sparsity (B=1, H=12, N=32760 = 21x30x52,
d=128, kh=5%, kl=10%).

Prints ONE JSON line: dense-equivalent throughput 4*B*H*N^2*d / t (the pages'
FLOPS = O(full attention)/t, SLA paper summary, section 5 "Efficiency"),
ms per step, a roofline entry for the dominant kernel (block-sparse attention,
timed on every step of the timed region with HIP events recorded around it on
the stream it runs on), a per-stage breakdown from a separate pass with every
kernel bracketed, per-step median/p10/p90 with and without a cache flush
between steps (a further pass, outside the timed region), and the float64 CPU
oracle timed on a bounded sample of the same workload.

    python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--config 3] [--no-cpu]
                    [--variant sla2|sla1] [--phi softmax|elu1]

--variant sla1 times the SLA formulation instead (sla1_forward: no router, the
branches fused as O = O_s + Proj(O_l) with a seeded d x d Proj), --phi elu1
the ELU+1 feature map of the linear branch. --op soft_topk times SoftTop-k
(sla_soft_topk) on the compressed logits of the workload instead of the
forward pass, and prints that op's own line; --op backward times the
backward pass (sla_backward) for the forward's mask and a seeded dO, and
--op backward --saved the backward from the state a saving forward pass
(sla_forward_train) kept (sla_backward_saved), which does not run the
forward again.
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
# The pages' SLA forward kernel at 95% sparsity on the Wan2.1-1.3B shape (SLA
# paper summary, Fig. 6): measured on another GPU (the same study times on an
# RTX5090), so it is reported as context beside the line, never divided into it.
PAGES_TFLOPS = 2996.0
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_8BIT_TFLOPS = 5000.0  # MI355X dense fp8 MFMA (int8: 5.0 POP/s)
PEAK_HBM_GBS = 8000.0
KERNELS = ["pool_proj", "score_select", "hz", "linear_sum", "sparse_attn_mix"]
KERNEL_SOURCES = {"sparse_attn_mix": "k_sparse.hip", "hz": "k_hz.hip", "linear_sum": "k_linear.hip",
                  "pool_proj": "k_pool.hip", "score_select": "k_select.hip"}


# ----------------------------------------------------------------- FLOP accounting

def dense_flops(B, H, N, d):
    """Dense attention: two N x N x d products per head, 2mnk each."""
    return 4.0 * B * H * N * N * d


def sparse_tile_flops(B, H, Nb, n_h, d):
    """Executed MFMA work of the sparse branch: n_h whole 64x64 tiles per query
    block, each S = Q K^T and O += P V (2 * 64*64*d flops apiece)."""
    return 4.0 * B * H * Nb * n_h * 64 * 64 * d


def sparse_kernel_flops(B, H, Nb, n_h, d, proj=False):
    """Algorithmic flops of the sparse-attention kernel per launch: the critical
    tiles plus the linear-branch output phi(Q_i) [H_i | Z_i] of every query block,
    and with proj (the SLA fusion) the d x d output map applied to O_l."""
    f = sparse_tile_flops(B, H, Nb, n_h, d) + 2.0 * B * H * Nb * 64 * d * (d + 1)
    return f + (2.0 * B * H * Nb * 64 * d * d if proj else 0.0)


def pages_flop_fraction(kh, N, d):
    """The pages' accounting of SLA's attention FLOPs relative to full attention:
    kh of the dense work plus the linear branch, 2*N*d^2 per head
    (SLA paper summary, Tables 1-2: SLA 2.73T/2.74T of 52.75T at kh=5%, Linear
    Only 0.10T, Top-10% 5.38T, Top-20% 10.65T)."""
    return kh + (2.0 * N * d * d) / (4.0 * N * N * d)


def kernel_bytes(B, H, N, d, Nb, n_h, quant=False):
    """Compulsory HBM bytes of each bf16 kernel per launch (each tensor once).
    With the 8-bit sparse branch the h/z stage also writes int8 K and its key
    bias (from the K rows it reads anyway) and fp8 V^T (the bf16 sparse kernel
    reads the V rows themselves), and the sparse kernel reads those 8-bit tiles."""
    X = 2.0 * B * H * N * d
    BH = B * H
    NN = d * d + d
    Nbp = (Nb + 31) // 32 * 32
    hx = 2.0 * BH * Nbp * NN
    Hx = 2.0 * BH * Nb * NN
    X8 = BH * Nb * 64 * d * 1.0     # one 8-bit copy, whole blocks
    kbias = 4.0 * BH * Nb * 64
    if quant:
        return {
            "pool_proj": 2 * X + 2 * 8.0 * BH * Nb * d,
            "score_select": 2 * 8.0 * BH * Nb * d + BH * Nb * Nb,
            "hz": 2 * X + hx + X8 + X8 + kbias,
            "linear_sum": hx + Hx + BH * Nb * Nb,
            "sparse_attn_mix": X + X8 + kbias + X8 + Hx + X,
        }
    return {
        "pool_proj": 2 * X + 2 * 8.0 * BH * Nb * d,
        "score_select": 2 * 8.0 * BH * Nb * d + BH * Nb * Nb,
        # K and V read, h_j and z_j written
        "hz": 2 * X + hx,
        "linear_sum": hx + Hx + BH * Nb * Nb,
        "sparse_attn_mix": X + X + X + Hx + X,  # Q, K tiles, V tiles, H_i, O (K/V once each)
    }


# --------------------------------------------------------------------- helpers

def _source_sha(name):
    path = os.path.join(ROOT, "sparse_linear_attention_block_amd", "csrc", name)
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def _traffic_from_profile(kernel, workload, source):
    """HBM bytes per launch from a committed counter summary of the same kernel
    source and workload, or None."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_hbm_counters.json")
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            rec = json.load(f)
        if rec.get("source_sha") != _source_sha(source):
            return None
        return float(rec["bytes_per_launch"])
    except (OSError, ValueError, KeyError):
        return None


def cpu_model() -> str:
    """The host CPU's model name from /proc/cpuinfo (or platform's guess)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or platform.machine()


def cpu_baseline(cfg, x, seconds, phi="softmax", proj_o=None):
    """The float64 oracle as it stands, on one head: its mask (router, pooling,
    scores, ranking) and the outputs of evenly spaced query blocks until about
    `seconds` of wall time; reported as dense-equivalent TFLOP/s of the sample.
    With proj_o, the SLA formulation (no router, O = O_s + O_l proj_o)."""
    import threadpoolctl
    import oracle as orc

    Nb = cfg.Nb
    N, d = x.N, x.d
    info = threadpoolctl.threadpool_info()
    cores = max([p.get("num_threads", 1) for p in info] or [1])
    order = list(range(0, Nb, 7)) + [i for i in range(Nb) if i % 7]
    pq, pk = (None, None) if proj_o is not None else (x.proj_q, x.proj_k)
    po = None if proj_o is None else proj_o[0] if proj_o.dim() == 3 else proj_o
    t0 = time.perf_counter()
    ref = orc.forward(x.q[:1, :1], x.k[:1, :1], x.v[:1, :1], pq, pk, x.alpha[:1],
                      x.kh, x.kl, compute_outputs=False, feature=phi, proj_o=po)
    mask = ref.mask
    done = []
    for i in order:
        orc.forward(x.q[:1, :1], x.k[:1, :1], x.v[:1, :1], pq, pk, x.alpha[:1],
                    x.kh, x.kl, mask_in=mask, query_blocks={(0, 0): [i]}, feature=phi, proj_o=po)
        done.append(i)
        if time.perf_counter() - t0 > seconds and len(done) >= 4:
            break
    dt = time.perf_counter() - t0
    toks = sum(min(64, N - 64 * i) for i in done)
    flops = 4.0 * toks * N * d
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s (dense-equivalent)", "cores": int(cores),
            "kind": "oracle", "cpu": cpu_model(),
            "sample": (f"{cfg.name}, head (0,0): router/pooling/scores/ranking of all {Nb} query-block "
                       f"rows plus explicit O(N^2) outputs of {len(done)} of {Nb} query blocks "
                       f"({toks} of {cfg.B * cfg.H * N} query tokens) in {dt:.1f} s; the rate is the "
                       f"sample's share of 4*B*H*N^2*d over its wall time"),
            "seconds": dt}


# SoftTop-k's search loop costs, per element and halving, 4 full-rate VALU ops
# (subtract, scale, add, accumulate; 64 lanes per CU per clock) and 2
# transcendental ones (exp2, reciprocal; 32 lanes per CU per clock on gfx950,
# twice CDNA3's rate): 4/64 + 2/64 * 2 = 0.125 CU-clocks, so the chip's 256
# CUs at 2.4 GHz evaluate at most 256 * 2.4e9 / 0.125 = 4.92e12 sigmoids per
# second.
PEAK_SIGMOID_PER_S = 256 * 2.4e9 / (4 / 64 + 2 / 32)


def soft_topk_halvings(P, lam, tau):
    """Halvings the float32 search makes per row: the bracket [min Pc - 60 tau,
    max Pc + 60 tau] halved towards the returned threshold until its float32
    midpoint stops moving."""
    lo = (P.min(axis=-1) - 60.0 * tau).astype(np.float32)
    hi = (P.max(axis=-1) + 60.0 * tau).astype(np.float32)
    lam = lam.astype(np.float32)
    n = np.zeros(lo.shape, dtype=np.int64)
    for _ in range(256):
        mid = np.float32(0.5) * (lo + hi)
        act = (mid > lo) & (mid < hi)
        if not act.any():
            break
        n += act
        up = act & (mid < lam)
        lo = np.where(up, mid, lo)
        hi = np.where(act & ~up, mid, hi)
    return n


def bench_soft_topk(args, cfg, x, torch, sla):
    """SoftTop-k over the workload's compressed logits (B*H*Nb rows of Nb),
    budget n_h, temperature --tau (Pc units); one JSON line."""
    import oracle as orc
    dev = torch.device("cuda:0")
    _, _, dbg = sla.forward(x.q.to(dev), x.k.to(dev), x.v.to(dev), x.proj_q.to(dev), x.proj_k.to(dev),
                            x.alpha.to(dev), x.kh, x.kl, debug=True)
    lg = dbg["logits"]
    B, H, Nb = lg.shape[0], lg.shape[1], lg.shape[2]
    rows = B * H * Nb
    n_h = sla.block_counts(x.N, x.kh, x.kl, B=B, H=H, d=x.d, dtype=cfg.dtype)[1]
    out = torch.empty(lg.shape, dtype=torch.float32, device=dev)
    lam = torch.empty(lg.shape[:-1], dtype=torch.float32, device=dev)
    for _ in range(args.warmup):
        sla.soft_topk(lg, n_h, args.tau, out=out, lam=lam)
    torch.cuda.synchronize()
    hev = sla.HipEvents()
    evs = hev.create(2 * args.steps)
    stream = torch.cuda.current_stream().cuda_stream
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for s in range(args.steps):
        hev.record(evs[2 * s], stream)
        sla.soft_topk(lg, n_h, args.tau, out=out, lam=lam)
        hev.record(evs[2 * s + 1], stream)
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps
    k_ms = float(np.mean([hev.elapsed_ms(evs[2 * s], evs[2 * s + 1]) for s in range(args.steps)]))
    hev.destroy(evs)
    lg_h = lg.cpu().numpy()
    P = orc.compressed_map(lg_h)
    halv = soft_topk_halvings(P, lam.cpu().numpy(), args.tau)
    evals = float(((halv + 1) * Nb).sum())  # every halving plus the output pass
    achieved = evals / (k_ms * 1e-3)
    line = {
        "metric": "SoftTop-k of the compressed attention map, rows per second",
        "value": round(rows / (ms * 1e-3), 1),
        "unit": "rows/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32 (float64 logits in)",
        "data": "the float64 compressed logits sla_forward computes for the seeded workload",
        "config": {"workload": cfg.name + "_soft_topk", "rows": rows, "cols": Nb, "k": n_h,
                   "tau": args.tau, "mean_halvings": round(float(halv.mean()), 2)},
        "roofline": {"kernel": "k_soft_topk", "bound": "alu", "achieved": round(achieved / 1e12, 4),
                     "peak": round(PEAK_SIGMOID_PER_S / 1e12, 4), "unit": "T sigmoid evaluations/s",
                     "frac": round(achieved / PEAK_SIGMOID_PER_S, 4), "traffic": None,
                     "ms_per_launch": round(k_ms, 5),
                     "hbm_bytes_per_launch": rows * Nb * 12 + rows * 4},
    }
    if not args.no_cpu:
        t0 = time.perf_counter()
        done = 0
        while time.perf_counter() - t0 < args.cpu_seconds and done < rows:
            orc.soft_topk(lg_h.reshape(rows, Nb)[done:done + 64], n_h, args.tau)
            done += 64
        dt = time.perf_counter() - t0
        import threadpoolctl
        cores = max([p.get("num_threads", 1) for p in threadpoolctl.threadpool_info()] or [1])
        line["cpu_baseline"] = {"value": round(done / dt, 1), "unit": "rows/s", "cores": int(cores),
                                "kind": "oracle", "cpu": cpu_model(),
                                "sample": f"the float64 oracle on the first {done} of {rows} rows "
                                          f"in {dt:.1f} s"}
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


# fp32 FMA on the VALU without packed operations: 64 lanes x 2 flops per CU
# per clock, 256 CUs at 2.4 GHz
PEAK_F32_VALU_TFLOPS = 256 * 64 * 2 * 2.4e9 / 1e12


def backward_flops(B, H, Nb, n_h, d):
    """Algorithmic flops of the backward pass: per (query block, critical tile)
    the five 64 x 64 x d products of the FlashAttention backward (S, dP, dV,
    dK, dQ), and per block the linear branch's five 64 x d x d products
    (num, du and dH_i on the query side, dw and dv on the key side)."""
    return 10.0 * B * H * Nb * n_h * 64 * 64 * d + 10.0 * B * H * Nb * 64 * d * d


def bench_backward(args, cfg, x, torch, sla, proj_o=None):
    """sla_backward (or, with proj_o, sla1_backward) at the workload's shape,
    for the mask its forward pass computes and a seeded dO; one JSON line."""
    from oracle import backward as ob
    dev = torch.device("cuda:0")
    q, k, v, al = x.q.to(dev), x.k.to(dev), x.v.to(dev), x.alpha.to(dev)
    sla1 = proj_o is not None
    saved = args.saved
    pq, pk = x.proj_q.to(dev), x.proj_k.to(dev)
    ws_saved = None
    if sla1:
        proj_o = proj_o.to(dev)
        if saved:
            _, mask, ws_saved = sla.forward_sla1_train(q, k, v, proj_o, x.kh, x.kl, proj_q=pq, proj_k=pk)
        else:
            _, mask = sla.forward_sla1(q, k, v, proj_o, x.kh, x.kl, proj_q=pq, proj_k=pk)
    else:
        if saved:
            _, mask, ws_saved = sla.forward_train(q, k, v, pq, pk, al, x.kh, x.kl)
        else:
            _, mask = sla.forward(q, k, v, pq, pk, al, x.kh, x.kl)
    g = np.random.default_rng(cfg.seed + 7).standard_normal(tuple(x.q.shape))
    dO = torch.from_numpy(g.astype(np.float32)).to(x.q.dtype)
    dO_d = dO.to(dev)
    B, H, N, d = x.q.shape
    Nb = cfg.Nb
    n_h = sla.block_counts(N, x.kh, x.kl, B=B, H=H, d=d, dtype=cfg.dtype)[1]
    p = sla.make_problem(B, H, N, d, cfg.dtype, 0.0, 0.0,
                         proj_head_stride=(d * d if sla1 and proj_o.dim() == 3 else 0))
    n = ctypes_size(sla, p, sla1)
    ws = torch.empty(n, dtype=torch.uint8, device=dev)

    if saved:
        # the saving forward's own cost, for the record (not part of the timed backward)
        def fwd_train():
            if sla1:
                sla.forward_sla1_train(q, k, v, proj_o, x.kh, x.kl, proj_q=pq, proj_k=pk, workspace=ws_saved)
            else:
                sla.forward_train(q, k, v, pq, pk, al, x.kh, x.kl, workspace=ws_saved)
        def fwd_plain():
            if sla1:
                sla.forward_sla1(q, k, v, proj_o, x.kh, x.kl, proj_q=pq, proj_k=pk)
            else:
                sla.forward(q, k, v, pq, pk, al, x.kh, x.kl)

        def per_call(fn):
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(10):
                fn()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / 10
        print(f"[bench] saving forward ({'sla1_' if sla1 else 'sla_'}forward_train): {per_call(fwd_train):.4f} ms "
              f"per call; the plain forward through the same binding call: {per_call(fwd_plain):.4f} ms",
              file=sys.stderr, flush=True)

    def run():
        if saved:  # the state in ws_saved is only read, so every call sees the same inputs
            if sla1:
                sla.backward_sla1_saved(q, k, v, proj_o, mask, dO_d, ws_saved)
            else:
                sla.backward_saved(q, k, v, al, mask, dO_d, ws_saved)
        elif sla1:
            sla.backward_sla1(q, k, v, proj_o, mask, dO_d, workspace=ws)
        else:
            sla.backward(q, k, v, al, mask, dO_d, workspace=ws)
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        run()
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps
    # the SLA fusion adds the output map's two products per token: dO_l = dO W^T and dW = O_l^T dO
    F = backward_flops(B, H, Nb, n_h, d) + (4.0 * B * H * N * d * d if sla1 else 0.0)
    achieved = F / (ms * 1e-3) / 1e12
    # bf16 inputs: every product on bf16 MFMA (float32 accumulation); float32 inputs: the VALU kernels
    mfma = cfg.dtype == "bf16"
    peak = PEAK_BF16_TFLOPS if mfma else PEAK_F32_VALU_TFLOPS
    line = {
        "metric": ("SLA" if sla1 else "SLA2") + " backward ms & dense-equivalent TFLOPS (10*B*H*N^2*d per backward)",
        "value": round(10.0 * B * H * N * N * d / (ms * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s (dense-equivalent backward)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16 MFMA, f32 accumulate" if mfma else "f32 (" + cfg.dtype + " inputs)",
        "data": "synthetic: the seeded workload, its forward mask and a seeded N(0,1) dO",
        "config": {"workload": cfg.name + ("_sla1" if sla1 else "") + "_backward" + ("_saved" if saved else ""),
                   "B": B, "H": H, "N": N, "d": d, "Nb": Nb,
                   "n_h": n_h, "kh": x.kh, "kl": x.kl},
        "roofline": {"kernel": ("sla1_backward" if sla1 else "sla_backward") + ("_saved" if saved else "")
                               + " (all its kernels)",
                     "bound": "mfma" if mfma else "alu",
                     "achieved": round(achieved, 3), "peak": round(peak, 1),
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": None, "flops_per_launch": F, "ms_per_launch": round(ms, 4)},
    }
    if not args.no_cpu and not sla1:
        import threadpoolctl
        cores = max([pp.get("num_threads", 1) for pp in threadpoolctl.threadpool_info()] or [1])
        mk = mask.cpu().numpy()
        t0 = time.perf_counter()
        done = 0
        for i in range(0, Nb, 7):
            ob.dq_rows(x.q, x.k, x.v, x.alpha, mk, dO, 0, 0, [i])
            done += 1
            if time.perf_counter() - t0 > args.cpu_seconds and done >= 2:
                break
        dt = time.perf_counter() - t0
        line["cpu_baseline"] = {
            "value": round(10.0 * 64 * N * d * done / dt / 1e12, 6), "unit": "TFLOP/s (dense-equivalent backward)",
            "cores": int(cores), "kind": "oracle", "cpu": cpu_model(),
            "sample": f"{cfg.name}, head (0,0): the float64 autograd oracle's dQ for {done} of {Nb} query "
                      f"blocks in {dt:.1f} s, counted as 10*64*N*d per block (dK and dV are not formed "
                      f"by this sample, so the rate flatters the oracle)"}
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


def ctypes_size(sla, p, sla1=False):
    import ctypes
    n = ctypes.c_size_t()
    lib = sla.load_library()
    fn = lib.sla1_backward_workspace_bytes if sla1 else lib.sla_backward_workspace_bytes
    rc = fn(ctypes.byref(p), ctypes.byref(n))
    if rc != 0:
        raise RuntimeError("sla_backward_workspace_bytes failed")
    return max(int(n.value), 256)


def step_distribution(torch, plan, hev, steps, flush_mib):
    """Per-step times after the timed region: each step bracketed by two
    fence-free HIP events on its stream. The unflushed steps run back to back;
    the flushed ones each follow a write of flush_mib MiB (outside the events),
    which evicts the L2 and the MALL. Reported as median, p10 and p90 in ms."""
    stream = torch.cuda.current_stream().cuda_stream

    def run(flush):
        evs = hev.create(2 * steps)
        for s in range(steps):
            if flush is not None:
                flush.fill_(s & 0xFF)
            hev.record(evs[2 * s], stream)
            plan.run()
            hev.record(evs[2 * s + 1], stream)
        torch.cuda.synchronize()
        t = np.array([hev.elapsed_ms(evs[2 * s], evs[2 * s + 1]) for s in range(steps)])
        hev.destroy(evs)
        return [round(float(np.percentile(t, q)), 5) for q in (50, 10, 90)]

    out = {"steps": steps}
    out["median"], out["p10"], out["p90"] = run(None)
    if flush_mib > 0:
        buf = torch.empty(flush_mib * 2 ** 20, dtype=torch.uint8, device="cuda")
        out["flush_mib"] = flush_mib
        out["flushed_median"], out["flushed_p10"], out["flushed_p90"] = run(buf)
        del buf
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--variant", choices=["sla2", "sla1"], default="sla2",
                    help="sla2: router + alpha mix (sla_forward); sla1: no router, "
                         "O = O_s + Proj(O_l) (sla1_forward)")
    ap.add_argument("--phi", choices=["softmax", "elu1"], default="softmax",
                    help="feature map of the linear branch")
    ap.add_argument("--op", choices=["forward", "soft_topk", "backward"], default="forward",
                    help="forward: the whole forward pass; soft_topk: SoftTop-k on its logits; "
                         "backward: the backward pass")
    ap.add_argument("--saved", action="store_true",
                    help="with --op backward: time the backward from a saving forward's state "
                         "(sla_forward_train, then sla_backward_saved)")
    ap.add_argument("--linear", choices=["gemm", "chain"], default="gemm",
                    help="marginal sums: gemm (indicator product per head) or chain (row-to-row updates)")
    ap.add_argument("--tau", type=float, default=1e-3, help="SoftTop-k temperature (Pc units)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--flush-mib", type=int, default=512,
                    help="MiB written between the flushed per-step timings (0: no flushed pass)")
    ap.add_argument("--settle-s", type=float, default=1.0,
                    help="seconds of back-to-back steps before the warm-up, so that the timed steps run at "
                         "the clock the chip holds under this load (a few warm-up steps alone leave it "
                         "ramping: 0.795 against 0.727 ms/step at the Wan2.1-1.3B shape)")
    ap.add_argument("--hbm-calib-mib", type=int, default=0,
                    help="before the warm-up, copy a buffer of this many MiB three times "
                         "(a plain copy kernel of known size, to scale HBM counters)")
    args = ap.parse_args()
    if args.saved and args.op != "backward":
        print("--saved applies to --op backward only", file=sys.stderr)
        sys.exit(2)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the SLA2 forward pass is built and timed on a "
              "single MI355X (heads shard across GPUs with no exchange; see the design notes).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import sparse_linear_attention_block_amd as sla
    from workloads import CONFIGS, make_inputs, make_proj_o

    cfg = CONFIGS[args.config]
    sla1 = args.variant == "sla1"
    if cfg.quant and sla1:
        print("the SLA formulation is built without the 8-bit sparse branch", file=sys.stderr)
        sys.exit(2)
    if cfg.quant:
        print("note: the 8-bit sparse branch is timed with quant=True", file=sys.stderr)
    # the name the profiles of this workload are filed under
    wl_name = (cfg.name + ("_sla1" if sla1 else "") + ("_elu1" if args.phi == "elu1" else "")
               + ("_chain" if args.linear == "chain" else ""))
    t0 = time.time()
    x = make_inputs(cfg)
    print(f"[bench] inputs {cfg.name} generated in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    if args.op == "soft_topk":
        bench_soft_topk(args, cfg, x, torch, sla)
        return
    if args.op == "backward":
        if cfg.quant:
            print("the backward pass is built without the 8-bit branch", file=sys.stderr)
            sys.exit(2)
        bench_backward(args, cfg, x, torch, sla, make_proj_o(cfg) if sla1 else None)
        return
    dev = torch.device("cuda:0")
    q, k, v = x.q.to(dev), x.k.to(dev), x.v.to(dev)
    # a workload whose router is the identity passes none (the block means are compared as
    # they are: the same pooled vectors, without an identity product)
    if cfg.router == "identity":
        pq = pk = None
    else:
        pq, pk = x.proj_q.to(dev), x.proj_k.to(dev)
    al = x.alpha.to(dev)
    proj_o = make_proj_o(cfg) if sla1 else None
    if sla1:
        plan = sla.Plan(q, k, v, None, None, None, x.kh, x.kl, phi=args.phi, proj_o=proj_o.to(dev),
                        linear=args.linear)
    else:
        plan = sla.Plan(q, k, v, pq, pk, al, x.kh, x.kl, quant=cfg.quant, phi=args.phi, linear=args.linear)
    B, H, N, d, Nb = plan.dims
    _, n_h, n_l = sla.block_counts(N, x.kh, x.kl, B=B, H=H, d=d, dtype=cfg.dtype)
    if args.hbm_calib_mib > 0:
        src = torch.ones(args.hbm_calib_mib * 2 ** 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] calibration copy: 3 x {args.hbm_calib_mib} MiB read + written",
              file=sys.stderr, flush=True)
        del src, dst

    settle_steps = 0
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < args.settle_s:
        for _ in range(10):
            plan.run()
        settle_steps += 10
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        plan.run()
    torch.cuda.synchronize()

    hev = sla.HipEvents()
    # Timed region: K whole steps; on every step the sparse kernel (the
    # roofline's kernel) is bracketed by two fence-free HIP events on its stream.
    evs = [hev.create(2) for _ in range(args.steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for s in range(args.steps):
        plan.run(events=[None, None, None, None, evs[s][0], evs[s][1]])
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps
    k5_ms = float(np.mean([hev.elapsed_ms(e[0], e[1]) for e in evs]))
    for e in evs:
        hev.destroy(e)
    # Stage breakdown, after the timed region: every kernel bracketed (each
    # event adds a little dispatch latency, so these steps are not the ones timed).
    nb = min(args.steps, 20)
    bevs = [hev.create(6) for _ in range(nb)]
    for s in range(nb):
        plan.run(events=bevs[s])
    torch.cuda.synchronize()
    per_kernel = {name: float(np.mean([hev.elapsed_ms(e[i], e[i + 1]) for e in bevs]))
                  for i, name in enumerate(KERNELS)}
    for e in bevs:
        hev.destroy(e)
    dist = step_distribution(torch, plan, hev, min(args.steps, 50), args.flush_mib)

    F = dense_flops(B, H, N, d)
    value = F / (ms * 1e-3) / 1e12
    k5_flops = sparse_kernel_flops(B, H, Nb, n_h, d, proj=sla1)
    achieved = k5_flops / (k5_ms * 1e-3) / 1e12
    peak = PEAK_8BIT_TFLOPS if cfg.quant else PEAK_BF16_TFLOPS
    k5_src = "k_sparse_q8.hip" if cfg.quant else KERNEL_SOURCES["sparse_attn_mix"]
    traffic = _traffic_from_profile("sparse_attn_mix", wl_name, k5_src)
    kb = kernel_bytes(B, H, N, d, Nb, n_h, cfg.quant)
    gbs = {name: kb[name] / (per_kernel[name] * 1e-3) / 1e9 for name in KERNELS}
    print(f"[bench] {wl_name}: {ms:.3f} ms/step, per kernel (ms) " +
          ", ".join(f"{n}={t:.4f}" for n, t in per_kernel.items()), file=sys.stderr, flush=True)

    line = {
        "metric": "sparse-linear attn fwd ms & dense-equiv TFLOPS, Wan-1.3B shape, 95/97% sparse",
        "value": round(value, 2),
        "unit": "TFLOP/s (dense-equivalent, 4*B*H*N^2*d per forward)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle": {"seconds": args.settle_s, "steps": settle_steps,
                   "note": "untimed back-to-back steps before the warm-up, for steady clocks"},
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("i8+fp8 (sparse branch), bf16 (linear branch)" if cfg.quant
                  else "bf16" if cfg.dtype == "bf16" else "f32"),
        "data": "synthetic: seeded video-DiT-shaped Q/K/V (3-axis sin/cos position field + noise), "
                "calibrated to the pages' attention-weight shares",
        "config": {"workload": wl_name, "B": B, "H": H, "N": N, "d": d, "kh": x.kh, "kl": x.kl,
                   "Nb": Nb, "n_h": n_h, "n_l": n_l, "quant": cfg.quant,
                   "sparsity": round(1 - n_h / Nb, 4),
                   "formulation": ("SLA: no router, O = O_s + Proj(O_l)" if sla1
                                   else "SLA2: O = alpha O_s + (1 - alpha) O_l, "
                                        + ("identity router (none applied: the block means are compared)"
                                           if cfg.router == "identity"
                                           else "learned router matrices I + 0.1 N(0, 1/d)")),
                   "phi": args.phi, "linear_sums": args.linear},
        "roofline": {"kernel": "sparse_attn_mix", "bound": "mfma", "achieved": round(achieved, 2),
                     "peak": peak, "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": traffic, "flops_per_launch": k5_flops, "ms_per_launch": round(k5_ms, 5)},
        "step_distribution": dist,
        "kernels_ms": {n: round(t, 5) for n, t in per_kernel.items()},
        "kernels_hbm_gbs": {n: round(t, 1) for n, t in gbs.items()},
    }
    if args.config == 3 and not sla1 and args.phi == "softmax":
        line["context"] = {"pages_sla_kernel_tflops": PAGES_TFLOPS,
                           "note": "the pages' SLA forward kernel at 95% sparsity on this shape, "
                                   "measured on another GPU; context, not a baseline"}
    if not args.no_cpu:
        cb = cpu_baseline(cfg, x, args.cpu_seconds, args.phi, proj_o)
        cb["value"] = round(cb["value"], 5)
        cb["seconds"] = round(cb["seconds"], 2)
        line["cpu_baseline"] = cb
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
