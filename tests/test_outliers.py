"""Host-side checks of the outlier-suppression tool (no GPU): its Sylvester matrix, its
Walsh-Hadamard transform, its column discrepancy (Definition 2.2 as read: the largest
absolute column sum of the +-1 matrix) and its int4 rule, against library routines, closed
forms and the oracle."""
import numpy as np
import pytest
import scipy.linalg
import torch

from oracle import convrot_oracle as O
from rotation_w4a4_quantized_convrot_amd import outliers as T


@pytest.mark.parametrize("n", [1, 2, 4, 16, 64, 256, 1024])
def test_sylvester_is_scipy_hadamard(n):
    assert np.array_equal(T.sylvester_pm1(n), scipy.linalg.hadamard(n))


@pytest.mark.parametrize("n", [4, 16, 256])
def test_fwht_matches_dense(n):
    x = torch.from_numpy(np.random.default_rng(n).standard_normal((5, 3, n)))
    ref = x.numpy() @ scipy.linalg.hadamard(n).T.astype(np.float64)
    assert np.allclose(T.fwht(x).numpy(), ref, rtol=0, atol=1e-12 * n)


@pytest.mark.parametrize("g", [4, 16, 64, 256, 1024])
def test_column_discrepancy_regular_vs_sylvester(g):
    # regular: every column sums to sqrt(g); Sylvester: column 0 sums to g, the rest to 0
    assert T.column_discrepancy(O.regular_hadamard(g)) == pytest.approx(np.sqrt(g), abs=0)
    assert T.column_discrepancy(T.sylvester_pm1(g)) == g


def test_column_discrepancy_lower_bound():
    # Theorem 2.1: the squared column sums of any H-matrix add up to n^2, so the largest is at
    # least sqrt(n); Hadamard matrices equivalent to Sylvester's (signed rows and columns)
    rng = np.random.default_rng(5)
    for n in (4, 16, 64):
        h = T.sylvester_pm1(n) * rng.choice([-1, 1], size=(n, 1)) * rng.choice([-1, 1], size=n)
        h = h[rng.permutation(n)][:, rng.permutation(n)]
        assert np.array_equal(h @ h.T, n * np.eye(n, dtype=np.int64))
        assert np.sum(h.sum(axis=0) ** 2) == n * n
        assert T.column_discrepancy(h) >= np.sqrt(n)


def test_sylvester_concentrates_a_constant_row():
    # a token with the same value c in every channel: Sylvester piles it into one entry
    # (c sqrt(g)); the regular transform leaves c everywhere
    c, g = 3.0, 256
    x = torch.full((1, g), c, dtype=torch.float64)
    y = T.sylvester_groups(x, g)
    assert float(y.abs().max()) == pytest.approx(c * np.sqrt(g))
    assert int((y.abs() > 1e-9).sum()) == 1
    assert np.allclose(O.rotate_groups(x.numpy(), g), c)
