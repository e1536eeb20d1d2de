"""CPU model of the solve kernel's elimination order (csrc/vda.hip, vda_solve_kernel).

The kernel inverts I + A (A = beta K^T K, symmetric positive semidefinite) by
Gauss-Jordan elimination of [I + A | I], one column per thread, rows rotated
so that the pivot row is always slot 0, and it never broadcasts the pivot
column: each thread publishes only its own pivot-row entry, the right half
negated, at position (c - k) mod 2d, and slots 0 .. d-1 of that buffer are
taken as the pivot column.  That rests on the symmetry of the Schur
complement that remains to be eliminated; this test runs the same steps on
the CPU (fp64 and fp32) and compares with numpy's inverse.  The GPU kernel
itself is covered by the state parity tests.
"""
import numpy as np
import pytest


def solve_like_kernel(a_mat, dtype):
    d = a_mat.shape[0]
    aug = np.concatenate([np.eye(d) + a_mat, np.eye(d)], axis=1).astype(dtype)
    cols = [aug[:, c].copy() for c in range(2 * d)]      # column c, slot s = row (k + s) mod d
    for k in range(d):
        buf = np.zeros(2 * d, dtype=dtype)
        for c in range(2 * d):
            buf[(c - k) % (2 * d)] = cols[c][0] if c < d else -cols[c][0]
        for c in range(2 * d):
            x = cols[c][0] / buf[0]
            new = np.empty(d, dtype=dtype)
            new[:d - 1] = cols[c][1:] - buf[1:d] * x
            new[d - 1] = x
            cols[c] = new
    return np.stack([cols[d + j] for j in range(d)], axis=1)


@pytest.mark.parametrize("d", [4, 8, 16])
def test_rotated_gauss_jordan_with_the_pivot_column_from_the_pivot_row(d):
    g = np.random.default_rng(d)
    k = g.normal(size=(2 * d, d))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    a = 0.8 * k.T @ k
    ref = np.linalg.inv(np.eye(d) + a)
    np.testing.assert_allclose(solve_like_kernel(a, np.float64), ref, rtol=0, atol=1e-13)
    np.testing.assert_allclose(solve_like_kernel(a, np.float32), ref, rtol=0, atol=1e-6)


def test_rank_deficient_and_zero_write_strength():
    """beta = 0 (A = 0) gives the identity; a rank-one A stays exact."""
    d = 8
    np.testing.assert_allclose(solve_like_kernel(np.zeros((d, d)), np.float64), np.eye(d), atol=0)
    v = np.arange(1, d + 1, dtype=np.float64)[:, None] / d
    a = v @ v.T
    ref = np.eye(d) - a / (1.0 + float((v.T @ v)[0, 0]))    # Sherman-Morrison
    np.testing.assert_allclose(solve_like_kernel(a, np.float64), ref, rtol=0, atol=1e-14)
