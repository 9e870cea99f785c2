"""Pins of the oracle's block Walsh-Hadamard rotation R = blockdiag(H_b) D / sqrt(b):
Sylvester's H_b against scipy's Hadamard construction (a library routine), the
algebra that makes it a rotation (orthogonal, H_b^2 = b I, the transform of a unit
vector), and the properties GPTQ relies on when it composes with the rotation (ork-driver
wiki "Exp 2026-08-18 GPTQ Int4": rotate, then quantise): outputs W X^T unchanged,
the Hessian's spectrum unchanged, and the PSD projection commuting with it."""
import numpy as np
import pytest
import scipy.linalg


@pytest.mark.parametrize("b", [1, 2, 4, 8, 64, 1024])
def test_sylvester_matches_scipy(orc, b):
    assert np.array_equal(orc.sylvester_hadamard(b), scipy.linalg.hadamard(b))


@pytest.mark.parametrize("K,b", [(8, 8), (96, 32), (1024, 256), (12, 4), (5, 1)])
def test_rotation_algebra(orc, K, b):
    s = np.random.default_rng(K + b).choice([-1.0, 1.0], K)
    R = orc.hadamard_rotation(K, b, s)
    assert np.allclose(R @ R.T, np.eye(K), atol=1e-12)
    Hb = orc.sylvester_hadamard(b)
    assert np.array_equal(Hb @ Hb, b * np.eye(b))
    # the transform of e_0 within a block is the first column of H_b / sqrt(b): all equal
    e = np.zeros(K)
    e[0] = 1.0
    y = orc.hadamard_rotation(K, b) @ e
    assert np.allclose(y[:b], 1 / np.sqrt(b)) and np.all(y[b:] == 0)
    # signs act on the input channels: R(s) = R(1) diag(s)
    assert np.allclose(R, orc.hadamard_rotation(K, b) * s[None, :])


def test_rotation_preserves_outputs_and_spectrum(orc):
    rng = np.random.default_rng(5)
    K, b = 256, 64
    W = rng.standard_normal((40, K)).astype(np.float32)
    X = rng.standard_normal((300, K)).astype(np.float32)
    s = rng.choice([-1.0, 1.0], K).astype(np.float32)
    Wr = orc.hadamard_rotate_rows(W, b, s)
    Xr = orc.hadamard_rotate_rows(X, b, s)
    assert np.allclose(Wr.astype(np.float64) @ Xr.T.astype(np.float64), W.astype(np.float64) @ X.T, rtol=0, atol=1e-3)
    H = orc.gram(X)
    Hr = orc.hadamard_rotate_hessian(H, b, s)
    assert np.allclose(np.linalg.eigvalsh(Hr.astype(np.float64)), np.linalg.eigvalsh(H.astype(np.float64)),
                       rtol=1e-5, atol=1e-3)
    # the Hessian of the rotated activations is the rotated Hessian
    assert np.allclose(orc.gram(Xr), Hr, rtol=1e-4, atol=1e-2)


def test_projection_commutes_with_rotation(orc):
    rng = np.random.default_rng(9)
    K, b = 128, 32
    A = rng.standard_normal((K, K))
    S = (A + A.T).astype(np.float32)                  # indefinite symmetric
    s = rng.choice([-1.0, 1.0], K)
    R = orc.hadamard_rotation(K, b, s)
    P1 = orc.psd_project(orc.hadamard_rotate_hessian(S, b, s)).astype(np.float64)
    P2 = R @ orc.psd_project(S).astype(np.float64) @ R.T
    assert np.linalg.norm(P1 - P2) / np.linalg.norm(P2) < 1e-5
