"""Float64 CPU fake-quantisation of the sparse branch in 8 bits (diagnosis only).

TEST INFRASTRUCTURE ONLY, like the rest of this package: imported by the
tests, never by the product path, and sharing no code with the HIP path.

It is NOT the pass criterion of the 8-bit path: the GPU's 8-bit sparse branch
is held to the unquantised float64 oracle (sla_oracle.sparse_branch) at
rel-L1 5e-2. This module gives the size of the error that quantisation alone
causes under the plainest reading of the pages, to tell a kernel bug from the
scheme's own error.

The SLA2 article (quantisation-aware paragraph) runs the sparse branch with
Q, K, P and V in 8 bits, each with a scale that is restored after the
product; the SLA2 cross-paper synthesis (section 3.3.1) names INT8 and FP8.
The pages give no format, scale granularity or rounding. The reading taken
here is the literal one:

* Q and K: symmetric int8, one scale per 64-token block:
  s = absmax / 127, code = round-half-even(x / s) clamped to [-127, 127].
* V: OCP fp8 e4m3 (finite, largest 448), one scale per 64-token block:
  s = absmax / 448, code = e4m3(x / s), round-half-even, saturating.
* A block whose entries are all zero has scale 1 (every code is 0).
* Scores from the codes: S = (q8 . k8) s_Q s_K / sqrt(d).
* P: for each query row and each critical 64-key tile, P~ = exp(S - m) with
  m the row's maximum score over its critical keys; s_P = max_tile(P~) / 448;
  P8 = e4m3(P~ / s_P). The tile adds s_P s_V * (P8 . v8) to the numerator.
  (P~ / s_P = 448 exp(S - max_tile S) does not depend on m.)
* The softmax denominator l sums the unquantised P~.
* O_s = numerator / l; zero for a query block with no critical block.

Codes are decided in float32 (the precision in which a GPU forms them);
everything after the codes is float64.

Pins (tests/test_oracle_quant.py): e4m3 against closed-form codes and the
torch float8_e4m3fn cast; int8 codes and scales; an exact case whose output is
the mean of V; an exact two-level case whose closed form holds only with one P
scale per tile; exact scaling by powers of two in V and in Q against K; with
the quantisers switched off it equals the unquantised sparse branch; its error
against that branch lies inside the 8-bit bar on N(0, 1) inputs.
"""

import numpy as np

from .sla_oracle import BLOCK, num_blocks

E4M3_MAX = 448.0
I8_MAX = 127.0


def e4m3(x) -> np.ndarray:
    """Nearest OCP e4m3 value (3 mantissa bits, exponent bias 7, subnormal
    spacing 2^-9), ties to even, after clamping to +-448."""
    x = np.clip(np.asarray(x, dtype=np.float64), -E4M3_MAX, E4M3_MAX)
    a = np.abs(x)
    _, E = np.frexp(a)                      # a = f * 2^E with f in [0.5, 1)
    e = np.maximum(E - 1, -6)               # binade exponent; subnormals share -6
    step = np.ldexp(1.0, e - 3)             # spacing of the binade's numbers
    q = np.rint(a / step) * step            # exact: division by a power of two
    return np.where(a == 0, 0.0, np.sign(x) * q)


def _block_scale(blk32: np.ndarray, top: float):
    """float32 absmax / top of one block (1 for an all-zero block) and the
    float32 multiplier top / absmax that forms the codes."""
    am = np.float32(np.abs(blk32).max()) if blk32.size else np.float32(0.0)
    if am > 0:
        return float(am / np.float32(top)), np.float32(top) / am
    return 1.0, np.float32(1.0)


def quant_i8_blocks(X: np.ndarray):
    """Symmetric int8 of X [N, d] per 64-token block: codes (float64 holding
    integers) and the block scales [Nb]."""
    N, d = X.shape
    X32 = np.asarray(X, dtype=np.float32)
    codes = np.zeros((N, d))
    scales = np.ones(num_blocks(N))
    for j in range(num_blocks(N)):
        blk = X32[j * BLOCK:(j + 1) * BLOCK]
        scales[j], inv = _block_scale(blk, I8_MAX)
        codes[j * BLOCK:(j + 1) * BLOCK] = np.clip(np.rint((blk * inv).astype(np.float32)), -I8_MAX, I8_MAX)
    return codes, scales


def quant_e4m3_blocks(X: np.ndarray):
    """e4m3 of X [N, d] per 64-token block: code values and block scales [Nb]."""
    N, d = X.shape
    X32 = np.asarray(X, dtype=np.float32)
    codes = np.zeros((N, d))
    scales = np.ones(num_blocks(N))
    for j in range(num_blocks(N)):
        blk = X32[j * BLOCK:(j + 1) * BLOCK]
        scales[j], inv = _block_scale(blk, E4M3_MAX)
        codes[j * BLOCK:(j + 1) * BLOCK] = e4m3((blk * inv).astype(np.float32))
    return codes, scales


def sparse_branch_q8(Q: np.ndarray, K: np.ndarray, V: np.ndarray, mask: np.ndarray,
                     query_blocks=None, quantize: bool = True) -> np.ndarray:
    """O_s of one head [N, d] with Q, K, V and P quantised as described above
    (rows of query blocks not asked for stay 0). mask: [Nb, Nb] in {1, 0, -1}.
    quantize=False keeps every value unrounded (unit scales), which must give
    the unquantised sparse branch."""
    N, d = Q.shape
    Nb = num_blocks(N)
    if quantize:
        q8, qs = quant_i8_blocks(Q)
        k8, ks = quant_i8_blocks(K)
        v8, vs = quant_e4m3_blocks(V)
        fp8 = e4m3
    else:
        q8, qs = np.asarray(Q, dtype=np.float64), np.ones(Nb)
        k8, ks = np.asarray(K, dtype=np.float64), np.ones(Nb)
        v8, vs = np.asarray(V, dtype=np.float64), np.ones(Nb)
        fp8 = lambda x: x
    out = np.zeros((N, d))
    for i in (range(Nb) if query_blocks is None else query_blocks):
        rows = slice(i * BLOCK, min((i + 1) * BLOCK, N))
        crit = [j for j in range(Nb) if mask[i, j] == 1]
        if not crit:
            continue
        tiles = []
        for j in crit:
            keys = slice(j * BLOCK, min((j + 1) * BLOCK, N))
            S = (q8[rows] @ k8[keys].T) * (qs[i] * ks[j]) / np.sqrt(d)
            tiles.append((j, keys, S))
        m = np.max([S.max(axis=1) for _, _, S in tiles], axis=0)[:, None]  # row max, critical keys
        num = np.zeros((rows.stop - rows.start, d))
        l = np.zeros((rows.stop - rows.start, 1))
        for j, keys, S in tiles:
            Pt = np.exp(S - m)                                      # P~
            l += Pt.sum(axis=1, keepdims=True)
            top = Pt.max(axis=1, keepdims=True)                    # 0 only if the tile underflows
            sP = np.where(top > 0, top / E4M3_MAX, 1.0) if quantize else np.ones_like(l)
            num += sP * vs[j] * (fp8(Pt / sP) @ v8[keys])
        out[rows] = num / l
    return out
