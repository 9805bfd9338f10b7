"""Pins of the oracle's int32 dot products (W2A8 page §三 item 2, §5.3).

Each check is independent of the oracle's own C loop: brute force in Python
integers, the +1/-1 split identity, closed-form special cases, and numpy's
int64 matmul (a library routine the oracle does not use).
"""
import itertools

import numpy as np
import pytest

import oracle


def test_brute_force_every_ternary_row_k8():
    # every one of the 3^8 ternary rows, against activation vectors that include the extremes
    K = 8
    w = np.array(list(itertools.product((-1, 0, 1), repeat=K)), dtype=np.int8)   # 6561 x 8
    g = np.random.Generator(np.random.PCG64(7))
    xs = [np.full(K, -128), np.full(K, 127), np.zeros(K), np.arange(K) - 4,
          np.array([-128, 127, -128, 127, 1, -1, 0, 5])]
    xs += [g.integers(-128, 128, size=K) for _ in range(4)]
    xq = np.array(xs, dtype=np.int8)                                             # 9 x 8
    acc = oracle.gemm_i32(xq, w)
    assert acc.shape == (len(xs), w.shape[0])
    wl = w.tolist()
    for m, x in enumerate(xq.tolist()):
        expect = [sum(a * b for a, b in zip(x, row)) for row in wl]
        assert acc[m].tolist() == expect


def test_plus_minus_identity():
    # sum_k a_k w_k = sum_{w=+1} a - sum_{w=-1} a, at a real layer size, several rows
    g = np.random.Generator(np.random.PCG64(11))
    M, N, K = 3, 300, 2560
    w = g.integers(-1, 2, size=(N, K), dtype=np.int8)
    xq = g.integers(-128, 128, size=(M, K), dtype=np.int8)
    acc = oracle.gemm_i32(xq, w)
    x64 = xq.astype(np.int64)
    for m in range(M):
        for n in range(N):
            plus = x64[m][w[n] == 1].sum()
            minus = x64[m][w[n] == -1].sum()
            assert acc[m, n] == plus - minus


def test_special_rows():
    g = np.random.Generator(np.random.PCG64(12))
    K = 1000
    xq = g.integers(-128, 128, size=(2, K), dtype=np.int8)
    w = np.zeros((5 + K // 100, K), dtype=np.int8)
    w[1] = 1
    w[2] = -1
    w[3, 17] = 1                      # one-hot +1
    w[4, 999] = -1                    # one-hot -1
    for i in range(K // 100):         # sparse rows with a single +1 at varying k
        w[5 + i, 100 * i + 3] = 1
    acc = oracle.gemm_i32(xq, w)
    sums = xq.astype(np.int64).sum(axis=1)
    assert (acc[:, 0] == 0).all()
    assert (acc[:, 1] == sums).all()
    assert (acc[:, 2] == -sums).all()
    assert (acc[:, 3] == xq[:, 17]).all()
    assert (acc[:, 4] == -xq[:, 999].astype(np.int32)).all()
    for i in range(K // 100):
        assert (acc[:, 5 + i] == xq[:, 100 * i + 3]).all()


def test_not_transposed_nonsquare():
    # M != N != K, so a transposed operand cannot even produce the right shape/values
    g = np.random.Generator(np.random.PCG64(13))
    xq = g.integers(-128, 128, size=(5, 48), dtype=np.int8)
    w = g.integers(-1, 2, size=(33, 48), dtype=np.int8)
    acc = oracle.gemm_i32(xq, w)
    assert acc.shape == (5, 33)
    ref = xq.astype(np.int64) @ w.astype(np.int64).T
    np.testing.assert_array_equal(acc, ref)


def test_matches_numpy_int64_matmul():
    g = np.random.Generator(np.random.PCG64(14))
    xq = g.integers(-128, 128, size=(4, 6912), dtype=np.int8)
    w = g.integers(-1, 2, size=(257, 6912), dtype=np.int8)
    np.testing.assert_array_equal(oracle.gemm_i32(xq, w),
                                  xq.astype(np.int64) @ w.astype(np.int64).T)


def test_empty_shapes():
    assert oracle.gemm_i32(np.zeros((1, 0), np.int8), np.zeros((3, 0), np.int8)).tolist() == [[0, 0, 0]]
    assert oracle.gemm_i32(np.zeros((0, 4), np.int8), np.zeros((3, 4), np.int8)).shape == (0, 3)


def test_int32_overflow_is_an_error():
    K = (1 << 24) + (1 << 20)          # 128 * K > 2^31
    xq = np.full((1, K), -128, dtype=np.int8)
    w = np.full((1, K), -1, dtype=np.int8)
    with pytest.raises(oracle.OracleError):
        oracle.gemm_i32(xq, w)
