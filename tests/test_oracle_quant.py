"""Pins of the 8-bit fake-quantised sparse branch (oracle/quant.py) on the CPU.

Each pin is fixed by the number formats or by exact arithmetic, not by the
module itself: the e4m3 codes by their definition and torch's cast, the int8
codes by their definition, whole outputs by inputs whose quantisation is
exact and whose result has a closed form.
"""

import numpy as np
import pytest
import torch

import oracle as orc
from oracle import quant as oq


def test_e4m3_closed_form_codes():
    # largest finite, smallest subnormal, ties to even in the normal and subnormal range
    cases = {448.0: 448.0, 460.0: 448.0, 1e6: 448.0, -470.0: -448.0,
             1.0625: 1.0, 1.1875: 1.25, 2.0 ** -9: 2.0 ** -9, 2.0 ** -10: 0.0,
             1.5 * 2.0 ** -10: 2.0 ** -9, 3 * 2.0 ** -10: 2 * 2.0 ** -9,
             2.0 ** -6: 2.0 ** -6, 0.0: 0.0, -0.3: -0.3125, 240.0: 240.0, 250.0: 256.0}
    for x, want in cases.items():
        assert oq.e4m3(x) == want, (x, oq.e4m3(x), want)


def test_e4m3_matches_torch_cast():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.uniform(-448, 448, 20000),
        rng.uniform(-1e-2, 1e-2, 20000),
        np.ldexp(rng.integers(-64, 64, 4000) + 0.5, rng.integers(-12, 3, 4000)),  # midpoints
    ]).astype(np.float32)
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(oq.e4m3(x), want)


def test_int8_codes_and_scales():
    X = np.zeros((70, 4), dtype=np.float32)
    X[0, 0] = 2.0          # block 0 absmax -> 127
    X[1, 1] = -2.0
    X[2, 2] = 2.0 * 2.5 / 127  # x * inv = 2.5 (up to f32) -> 2 (even) or 3
    X[3, 3] = 2.0 * 0.5 / 127
    codes, scales = oq.quant_i8_blocks(X)
    assert codes[0, 0] == 127 and codes[1, 1] == -127
    assert scales[0] == pytest.approx(2.0 / 127, rel=1e-7)
    assert scales[1] == 1.0 and not codes[64:].any()       # all-zero block
    inv = np.float32(127.0) / np.float32(2.0)
    assert codes[2, 2] == np.rint(np.float32(X[2, 2]) * inv)
    assert abs(codes[3, 3]) <= 1


# V entries whose e4m3 codes are exact: every block holds 1.75, so its scale is
# 1.75 / 448 = 2^-8 and the entries become 64, 128, 256 and 448
V_LEVELS = [-1.75, -1.0, -0.5, -0.25, 0.25, 0.5, 1.0, 1.75]


def _exact_v(N, d, seed):
    rng = np.random.default_rng(seed)
    V = rng.choice(V_LEVELS, size=(N, d))
    V[::64, 0] = 1.75
    return V


def test_exact_case_is_mean_of_v():
    # Q = 0: every score is 0, every P~ is 1 and every P8 is 448 exactly
    N, d = 300, 64
    rng = np.random.default_rng(1)
    Q = np.zeros((N, d))
    K = rng.standard_normal((N, d))
    V = _exact_v(N, d, 2)
    Nb = orc.num_blocks(N)
    mask = np.zeros((Nb, Nb), dtype=np.int8)
    mask[0, [0, 2, 4]] = 1
    mask[1, [1, 4]] = 1          # the ragged block (44 keys)
    mask[2, 3] = 1
    out = oq.sparse_branch_q8(Q, K, V, mask)
    for i, crit in ((0, [0, 2, 4]), (1, [1, 4]), (2, [3])):
        want = V[orc.token_rows(crit, N)].mean(axis=0)
        rows = orc.token_rows([i], N)
        np.testing.assert_allclose(out[rows], np.broadcast_to(want, (len(rows), d)), rtol=1e-14, atol=1e-15)
    assert not out[orc.token_rows([3], N)].any()   # no critical block: zero


def test_two_level_case_needs_one_p_scale_per_tile():
    """Two critical tiles whose scores are 0 and about -8: within a tile every
    P~ is the same, so with one P scale per row and tile every code is 448 and
    O_s is exactly (e^0 sum V_A + e^-8 sum V_B) / (64 (e^0 + e^-8)). One scale
    for the whole row would code tile B's P~ = 448 e^-8 = 0.150 as 0.15625 and
    miss the closed form by about 1e-5."""
    N, d = 192, 64
    Q = np.zeros((N, d))
    Q[:, 0] = 1.0                 # block absmax 1: code 127, scale fl32(1/127)
    K = np.zeros((N, d))
    K[128:192, 0] = -64.0         # block 2: code -127, scale fl32(64/127); block 1 stays 0
    V = _exact_v(N, d, 3)
    mask = np.array([[0, 1, 1], [0, 0, 0], [0, 0, 0]], dtype=np.int8)
    out = oq.sparse_branch_q8(Q, K, V, mask)
    s_b = 127.0 * float(np.float32(1.0) / np.float32(127.0)) * -127.0 * \
        float(np.float32(64.0) / np.float32(127.0)) / 8.0                   # about -8
    w_a, w_b = 1.0, np.exp(s_b)
    want = (w_a * V[64:128].sum(axis=0) + w_b * V[128:192].sum(axis=0)) / (64.0 * (w_a + w_b))
    np.testing.assert_allclose(out[:64], np.broadcast_to(want, (64, d)), rtol=1e-12, atol=1e-14)
    assert not out[64:].any()


def test_scales_exactly_with_powers_of_two():
    Q, K, V = _head(500, 64, 2)
    Nb = orc.num_blocks(500)
    mask = np.random.default_rng(3).choice([1, 0], size=(Nb, Nb), p=[0.4, 0.6]).astype(np.int8)
    a = oq.sparse_branch_q8(Q, K, V, mask)
    np.testing.assert_array_equal(oq.sparse_branch_q8(Q, K, V * 8.0, mask), a * 8.0)
    # Q up by 4 and K down by 4: the codes are unchanged and the scores too
    np.testing.assert_array_equal(oq.sparse_branch_q8(Q * 4.0, K * 0.25, V, mask), a)


def _head(N, d, seed):
    rng = np.random.default_rng(seed)
    bf = lambda a: torch.from_numpy(a.astype(np.float32)).bfloat16().double().numpy()
    return bf(rng.standard_normal((N, d))), bf(rng.standard_normal((N, d))), bf(rng.standard_normal((N, d)))


def _ref_sparse(Q, K, V, mask):
    N = Q.shape[0]
    ref = np.zeros_like(Q)
    for i in range(orc.num_blocks(N)):
        rows = orc.token_rows([i], N)
        ref[rows] = orc.sparse_branch(Q[rows], K, V, orc.token_mask(mask[i], 1, N))
    return ref


def test_without_rounding_is_the_sparse_branch():
    N, d = 700, 64
    Q, K, V = _head(N, d, 7)
    Nb = orc.num_blocks(N)
    mask = np.random.default_rng(8).choice([1, 0, -1], size=(Nb, Nb), p=[0.4, 0.4, 0.2]).astype(np.int8)
    mask[2] = -1
    got = oq.sparse_branch_q8(Q, K, V, mask, quantize=False)
    np.testing.assert_allclose(got, _ref_sparse(Q, K, V, mask), rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("d", [64, 128])
def test_close_to_unquantised(d):
    N = 640
    Q, K, V = _head(N, d, 4 + d)
    Nb = orc.num_blocks(N)
    mask = np.random.default_rng(5).choice([1, 0, -1], size=(Nb, Nb), p=[0.3, 0.5, 0.2]).astype(np.int8)
    mask[:, 0] = 1
    q8 = oq.sparse_branch_q8(Q, K, V, mask)
    ref = _ref_sparse(Q, K, V, mask)
    err = np.abs(q8 - ref).sum() / np.abs(ref).sum()
    assert 1e-3 < err < 5e-2, err     # quantisation is visible, within the 8-bit bar
