"""CPU checks of the model of the 8-bit kernel's arithmetic (tests/q8_kernel_model.py).

The model is a regression aid for the 8-bit kernel, not the oracle; these
checks make sure that it is itself right: e4m3 and int8 codes, an exact case,
exact scaling, and the unquantised branch when its quantisers are off.
"""

import numpy as np
import pytest
import torch

import oracle as orc
import q8_kernel_model as oq


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


def _head(N, d, seed):
    rng = np.random.default_rng(seed)
    bf = lambda a: torch.from_numpy(a.astype(np.float32)).bfloat16().double().numpy()
    return bf(rng.standard_normal((N, d))), bf(rng.standard_normal((N, d))), bf(rng.standard_normal((N, d)))


def test_branch_exact_case_is_mean_of_v():
    # Q = 0: every score is 0 and every P~ = 1, so each P8 is 448 exactly. With
    # absmax 1.75 every V scale is 1/256 (exact in float32) and the entries
    # +-0.25, +-0.5, +-1, +-1.75 become the e4m3 numbers 64, 128, 256, 448.
    N, d = 300, 64
    rng = np.random.default_rng(1)
    Q = np.zeros((N, d))
    K = rng.standard_normal((N, d))
    V = rng.choice([-1.75, -1.0, -0.5, -0.25, 0.25, 0.5, 1.0, 1.75], size=(N, d))
    V[::64, 0] = 1.75
    Nb = orc.num_blocks(N)
    mask = np.zeros((Nb, Nb), dtype=np.int8)
    mask[0, [0, 2, 4]] = 1       # odd count: the last pair holds one block
    mask[1, [1, 4]] = 1          # the ragged block in a pair
    mask[2, 3] = 1
    out = oq.sparse_branch_q8(Q, K, V, mask)
    for i, crit in ((0, [0, 2, 4]), (1, [1, 4]), (2, [3])):
        keys = orc.token_rows(crit, N)
        want = V[keys].mean(axis=0)
        rows = orc.token_rows([i], N)
        np.testing.assert_allclose(out[rows], np.broadcast_to(want, (len(rows), d)), rtol=1e-14, atol=1e-15)
    assert not out[orc.token_rows([3], N)].any()   # no critical block: zero


def test_branch_scales_exactly_with_v():
    Q, K, V = _head(500, 64, 2)
    Nb = orc.num_blocks(500)
    rng = np.random.default_rng(3)
    mask = rng.choice([1, 0], size=(Nb, Nb), p=[0.4, 0.6]).astype(np.int8)
    a = oq.sparse_branch_q8(Q, K, V, mask)
    b = oq.sparse_branch_q8(Q, K, V * 8.0, mask)
    np.testing.assert_array_equal(b, a * 8.0)


def _ref_sparse(Q, K, V, mask):
    N = Q.shape[0]
    ref = np.zeros_like(Q)
    for i in range(orc.num_blocks(N)):
        rows = orc.token_rows([i], N)
        ref[rows] = orc.sparse_branch(Q[rows], K, V, orc.token_mask(mask[i], 1, N))
    return ref


def test_branch_without_rounding_is_the_sparse_branch():
    # the smoothing split, the key bias, the pairs and the scale restore are exact algebra
    N, d = 700, 64
    Q, K, V = _head(N, d, 7)
    Q += 3.0 * np.sin(np.arange(N))[:, None] + 2.0     # a shared offset for the smoothing to remove
    K -= 1.5
    Nb = orc.num_blocks(N)
    rng = np.random.default_rng(8)
    mask = rng.choice([1, 0, -1], size=(Nb, Nb), p=[0.4, 0.4, 0.2]).astype(np.int8)
    mask[2] = -1
    got = oq.sparse_branch_q8(Q, K, V, mask, quantize=False)
    np.testing.assert_allclose(got, _ref_sparse(Q, K, V, mask), rtol=1e-5, atol=1e-6)


def test_branch_invariant_to_a_shared_key_offset():
    Q, K, V = _head(400, 64, 9)
    Nb = orc.num_blocks(400)
    mask = np.random.default_rng(10).choice([1, 0], size=(Nb, Nb), p=[0.5, 0.5]).astype(np.int8)
    a = oq.sparse_branch_q8(Q, K, V, mask)
    b = oq.sparse_branch_q8(Q, K + 0.5, V, mask)    # K - mean(K) is unchanged
    np.testing.assert_allclose(b, a, rtol=1e-6, atol=1e-6)


@pytest.mark.parametrize("d", [64, 128])
def test_branch_close_to_unquantised(d):
    N = 640
    Q, K, V = _head(N, d, 4 + d)
    Nb = orc.num_blocks(N)
    rng = np.random.default_rng(5)
    mask = rng.choice([1, 0, -1], size=(Nb, Nb), p=[0.3, 0.5, 0.2]).astype(np.int8)
    mask[:, 0] = 1
    q8 = oq.sparse_branch_q8(Q, K, V, mask)
    ref = _ref_sparse(Q, K, V, mask)
    err = np.abs(q8 - ref).sum() / np.abs(ref).sum()
    assert 1e-3 < err < 5e-2, err     # quantisation is visible, within the 8-bit bar
