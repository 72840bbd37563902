"""A model of the 8-bit sparse kernel's own arithmetic, on the CPU.

NOT THE ORACLE. This file restates, in float64 numpy, the choices the 8-bit
HIP kernel makes that the pages do not fix: Q/K smoothing by their channel
means, one P scale per query row and per PAIR of 64-key tiles (the unit of the
16x16x128 fp8 product), a power-of-two (E8M0) P scale, a softmax reference that
is an integer in log2 units. It exists so that a GPU test can tell a kernel
bug from the quantisation error of the scheme: the kernel should follow it up
to float32 rounding. It is a regression check of the kernel and nothing more;
the pass criterion of the 8-bit path is the unquantised float64 oracle
(oracle.sla_oracle) at rel-L1 5e-2, and the plain per-tile scheme of the pages'
reading lives in oracle/quant.py.

The scheme modelled here:

* Q and K are first smoothed by their channel means over the head's N
  tokens (q̄, k̄): q.k splits into (q - q̄).(k - k̄) + q̄.(k - k̄) + q.k̄, the
  last term is the same for every key of a query and cancels in the softmax,
  the middle one is a per-key bias kept in floating point, and only the
  first is quantised.
* Q - q̄ and K - k̄: symmetric int8, one scale per 64-token block,
  scale = absmax / 127, code = round-half-even(x * (127 / absmax)) clamped
  to +-127.
* V: OCP fp8 e4m3 (finite, max 448), one scale per 64-token block,
  scale = absmax / 448, code = e4m3(x * (448 / absmax)), round-half-even,
  saturating. An all-zero block has scale 1 (every code is 0).
* P: quantised per query row over the 128 keys of two consecutive critical
  key blocks (the critical list in ascending block order, taken in pairs; an
  odd last block forms a pair alone), after the V scale of each key's block is
  folded in: P' = P~ * s_V, s_P = 2^ceil(log2(rowmax(P') / 448)), the
  exponent kept in [-127, 127], P8 = e4m3(P' / s_P). P~ is taken against a
  reference that is an integer in log2 units.
* The softmax denominator sums the unquantised P~.

Codes are decided in float32 (the kernel's precision); everything after the
codes is float64.
"""

import numpy as np

from oracle.sla_oracle import BLOCK, num_blocks

E4M3_MAX = 448.0


def e4m3(x) -> np.ndarray:
    """Value of the nearest OCP e4m3 number (3 mantissa bits, exponent bias 7,
    subnormal step 2^-9), ties to even, after clamping to +-448."""
    x = np.clip(np.asarray(x, dtype=np.float64), -E4M3_MAX, E4M3_MAX)
    a = np.abs(x)
    _, E = np.frexp(a)                      # a = m * 2^E, m in [0.5, 1)
    e = np.maximum(E - 1, -6)               # exponent of the binade (subnormals share -6)
    step = np.ldexp(1.0, e - 3)             # spacing of e4m3 numbers in that binade
    q = np.rint(a / step) * step            # a / step is exact (power-of-two scaling)
    return np.where(a == 0, 0.0, np.sign(x) * q)


def quant_i8_blocks(X: np.ndarray):
    """Per-64-token-block symmetric int8 of X [N, d] (float32 values): codes
    (float64 holding integers) and scales [Nb]."""
    N, d = X.shape
    Nb = num_blocks(N)
    X32 = X.astype(np.float32)
    codes = np.zeros((N, d))
    scales = np.ones(Nb)
    for j in range(Nb):
        blk = X32[j * BLOCK:(j + 1) * BLOCK]
        am = np.float32(np.abs(blk).max()) if blk.size else np.float32(0)
        inv = np.float32(127.0) / am if am > 0 else np.float32(1.0)
        scales[j] = float(am / np.float32(127.0)) if am > 0 else 1.0
        c = np.rint((blk * inv).astype(np.float32))
        codes[j * BLOCK:(j + 1) * BLOCK] = np.clip(c, -127, 127)
    return codes, scales


def smooth(X: np.ndarray):
    """Channel mean of X [N, d] over its tokens (float32) and X - mean in float32."""
    mean = X.astype(np.float64).mean(axis=0).astype(np.float32)
    return mean, (X.astype(np.float32) - mean).astype(np.float32)


def quant_e4m3_blocks(X: np.ndarray):
    """Per-64-token-block e4m3 of X [N, d]: code values and scales [Nb]."""
    N, d = X.shape
    Nb = num_blocks(N)
    X32 = X.astype(np.float32)
    codes = np.zeros((N, d))
    scales = np.ones(Nb)
    for j in range(Nb):
        blk = X32[j * BLOCK:(j + 1) * BLOCK]
        am = np.float32(np.abs(blk).max()) if blk.size else np.float32(0)
        inv = np.float32(E4M3_MAX) / am if am > 0 else np.float32(1.0)
        scales[j] = float(am / np.float32(E4M3_MAX)) if am > 0 else 1.0
        codes[j * BLOCK:(j + 1) * BLOCK] = e4m3((blk * inv).astype(np.float32))
    return codes, scales


def sparse_branch_q8(Q: np.ndarray, K: np.ndarray, V: np.ndarray, mask: np.ndarray,
                     query_blocks=None, quantize: bool = True) -> np.ndarray:
    """O_s of one head [N, d] under the 8-bit scheme above (rows of the query
    blocks not asked for stay 0). mask [Nb, Nb] in {1, 0, -1}. With
    quantize=False every code is its unrounded value (scale 1), which must
    give the unquantised sparse branch."""
    N, d = Q.shape
    Nb = num_blocks(N)
    qm, qsm = smooth(Q)
    km, ksm = smooth(K)
    bias = ksm.astype(np.float64) @ qm.astype(np.float64)        # q̄.(k - k̄) per key
    if quantize:
        q8, qs = quant_i8_blocks(qsm)
        k8, ks = quant_i8_blocks(ksm)
        v8, vs = quant_e4m3_blocks(V)
        fp8 = e4m3
    else:
        q8, qs = qsm.astype(np.float64), np.ones(Nb)
        k8, ks = ksm.astype(np.float64), np.ones(Nb)
        v8, vs = V.astype(np.float64), np.ones(Nb)
        fp8 = lambda x: x
    out = np.zeros((N, d))
    blocks = range(Nb) if query_blocks is None else query_blocks
    for i in blocks:
        rows = slice(i * BLOCK, min((i + 1) * BLOCK, N))
        crit = [j for j in range(Nb) if mask[i, j] == 1]
        if not crit:
            continue
        # dequantised scores plus key bias for every critical key (natural log domain)
        segs = []
        for j in crit:
            keys = slice(j * BLOCK, min((j + 1) * BLOCK, N))
            s = ((q8[rows] @ k8[keys].T) * (qs[i] * ks[j]) + bias[keys][None, :]) / np.sqrt(d)
            segs.append((j, keys, s))
        # reference: the row maximum rounded up to an integer power of two
        m = np.ceil(max(s.max() for _, _, s in segs) / np.log(2.0)) * np.log(2.0)
        l = np.zeros((rows.stop - rows.start, 1))
        num = np.zeros((rows.stop - rows.start, d))
        for p in range(0, len(segs), 2):
            pair = segs[p:p + 2]
            pt = [np.exp(s - m) for _, _, s in pair]          # P~
            l += sum(x.sum(axis=1, keepdims=True) for x in pt)
            pp = [x * vs[j] for x, (j, _, _) in zip(pt, pair)]  # P' = P~ s_V
            pm = np.max(np.concatenate(pp, axis=1), axis=1, keepdims=True)
            if quantize:                                       # s_P = 2^E, E8M0 range
                E = np.ceil(np.log2(np.where(pm > 0, pm, 1.0) / E4M3_MAX))
                sp = np.ldexp(1.0, np.clip(E, -127, 127).astype(np.int64))
            else:
                sp = np.ones_like(pm)
            acc = np.zeros_like(num)
            for x, (_, keys, _) in zip(pp, pair):
                acc += fp8(x / sp) @ v8[keys]
            num += acc * sp
        out[rows] = num / l
    return out
