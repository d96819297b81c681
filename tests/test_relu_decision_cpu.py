"""The ReLU-gradient comparison used by the GPU parity tests, on the CPU.

ReLU's derivative is a decision on the sign of U; where |U| is within the
float32 accumulation bound either decision is correct.  Planted here: a
flipped decision on a sign-ambiguous element passes, a flipped decision on a
clear element fails, and an ambiguous element that is neither 0 nor dA
fails."""
import numpy as np
import pytest

import oracle
from tests.helpers import assert_relu_grad


def _case():
    rng = np.random.default_rng(3)
    N, h, F = 40, 64, 48
    X = rng.standard_normal((N, h))
    W1 = rng.standard_normal((h, F)) / 8
    # one pre-activation made exactly (numerically) zero: the sign of the
    # float32 sum there is anyone's guess
    X[5] = 0.0
    X[5, 0], X[5, 1] = 1.0, 1.0
    W1[0, 7], W1[1, 7] = 0.5, -0.5
    U = X @ W1
    dA = rng.standard_normal((N, F))
    dU = oracle.act_backward("relu", dA, U)
    return X, W1, U, dA, dU


def test_matching_result_passes():
    X, W1, U, dA, dU = _case()
    assert_relu_grad("dU", dU.copy(), dU, dA, X, W1)


def test_flip_on_a_sign_ambiguous_element_passes():
    X, W1, U, dA, dU = _case()
    assert U[5, 7] == 0.0
    g = dU.copy()
    g[5, 7] = dA[5, 7]              # the other valid decision
    assert_relu_grad("dU", g, dU, dA, X, W1)


def test_flip_on_a_clear_element_fails():
    X, W1, U, dA, dU = _case()
    i, j = np.unravel_index(np.argmax(np.abs(U) * (np.abs(dA) > 1)), U.shape)
    g = dU.copy()
    g[i, j] = dA[i, j] - dU[i, j]   # the wrong decision where the sign is clear
    with pytest.raises(AssertionError):
        assert_relu_grad("dU", g, dU, dA, X, W1)


def test_ambiguous_element_with_another_value_fails():
    X, W1, U, dA, dU = _case()
    g = dU.copy()
    g[5, 7] = dA[5, 7] + 2 * np.abs(dU).max()
    with pytest.raises(AssertionError):
        assert_relu_grad("dU", g, dU, dA, X, W1)


def test_small_dA_decision_is_followed_downstream():
    """Where dA itself is small, the GPU's positive decision (dU = dA) must
    still be taken into the reference for the gradients computed from dU:
    with one token, dW1 = x^T dU makes every column follow one decision."""
    X, W1, U, dA, dU = _case()
    dA = dA.copy()
    dA[5, 7] = 1e-3 * np.abs(dA).max()          # small, below the elementwise tolerance
    dU = oracle.act_backward("relu", dA, U)      # exact decision at U = 0: zero
    g = dU.copy()
    g[5, 7] = dA[5, 7]                           # the GPU decided positive
    ref = assert_relu_grad("dU", g, dU, dA, X, W1)
    assert ref[5, 7] == dA[5, 7]


def test_ambiguous_element_near_zero_but_not_zero_fails():
    """The zero decision is exactly zero in the GPU's epilogue (dA times 0),
    so a small nonzero value that is not dA is a wrong result."""
    X, W1, U, dA, dU = _case()
    dA = dA.copy()
    dA[5, 7] = np.abs(dA).max()                  # dA large: the two decisions far apart
    dU = oracle.act_backward("relu", dA, U)
    g = dU.copy()
    g[5, 7] = 1e-3 * np.abs(dA).max()            # neither exactly 0 nor near dA
    with pytest.raises(AssertionError):
        assert_relu_grad("dU", g, dU, dA, X, W1)


def test_dA_decision_error_counts_in_the_comparison():
    """At an element decided as dA the GPU value is compared, not replaced:
    a value off by more than the elementwise bound fails."""
    X, W1, U, dA, dU = _case()
    g = dU.copy()
    tol = 3e-2 * np.abs(dA).max()
    g[5, 7] = dA[5, 7] + 1.5 * tol
    with pytest.raises(AssertionError):
        assert_relu_grad("dU", g, dU, dA, X, W1)
