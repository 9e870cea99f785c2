"""CPU pins for the oracle's eigensolvers and PSD projection.

Page: hipfire-calib-data dataset card, section "The fix" (eigendecompose, clip
negative eigenvalues to zero, rebuild, symmetrise; 0.1004% change against bf16's
~0.391% step; Cholesky then succeeds at damp 0.01).
"""
import json
import os

import numpy as np
import pytest

import synthgen as g

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _sym(A):
    A = np.asarray(A, np.float64)
    return np.tril(A) + np.tril(A, -1).T


def _rand_sym(seed, K):
    rng = np.random.default_rng(seed)
    A = rng.standard_normal((K, K))
    return ((A + A.T) / 2).astype(np.float32)


@pytest.mark.parametrize("method", [0, 1])
def test_eigh_reconstructs_and_is_orthonormal(orc, method):
    H = _rand_sym(0, 96)
    w, V = orc.eigh(H, method)
    A = _sym(H)
    assert np.abs(V @ np.diag(w) @ V.T - A).max() < 1e-12
    assert np.abs(V.T @ V - np.eye(96)).max() < 1e-12


def test_jacobi_equals_tridiagonal_qr(orc):
    H = _rand_sym(1, 128)
    w0, V0 = orc.eigh(H, 0)
    w1, V1 = orc.eigh(H, 1)
    np.testing.assert_allclose(np.sort(w0), np.sort(w1), atol=1e-12)
    P0 = orc.psd_project(H, 0, return_f64=True)[1]
    P1 = orc.psd_project(H, 1, return_f64=True)[1]
    assert np.abs(P0 - P1).max() < 1e-12


def test_eigvalsh_matches_library_special_case(orc):
    """numpy's LAPACK eigvalsh as an independent library special case."""
    H = _rand_sym(2, 300)
    np.testing.assert_allclose(orc.eigvalsh(H), np.linalg.eigvalsh(_sym(H)), atol=1e-11)


def test_known_spectrum(orc):
    rng = np.random.default_rng(3)
    Q, _ = np.linalg.qr(rng.standard_normal((64, 64)))
    lam = np.linspace(-3, 5, 64)
    A = (Q * lam) @ Q.T
    w = orc.eigvalsh_f64(A)
    np.testing.assert_allclose(w, lam, atol=1e-12)


def test_psd_2x2_closed_form(orc):
    a, b, c = 1.0, 2.0, -0.5     # indefinite
    H = np.array([[a, b], [b, c]], np.float32)
    m, r = (a + c) / 2, np.hypot((a - c) / 2, b)
    lp = m + r                   # positive eigenvalue; the other is m - r < 0
    v = np.array([b, lp - a]); v /= np.linalg.norm(v)
    ref = lp * np.outer(v, v)
    P, P64 = orc.psd_project(H, 1, return_f64=True)
    assert np.abs(P64 - ref).max() < 1e-14


def test_psd_diagonal_input(orc):
    d = np.array([3.0, -1.0, 0.0, 2.5, -7.0], np.float32)
    P = orc.psd_project(np.diag(d))
    assert np.array_equal(P, np.diag(np.maximum(d, 0)).astype(np.float32))


def test_psd_of_psd_gram_is_unchanged(orc):
    wl = g.WORKLOADS["tiny"]
    H = orc.gram(g.x_chunk(wl)).astype(np.float32)
    P = orc.psd_project(H)
    assert np.linalg.norm(P - H) / np.linalg.norm(H) < 1e-6


def _kkt(orc, H, P64):
    """Projection onto the PSD cone is characterised by P >= 0, P - H >= 0 and
    <P, P - H> = 0 (the negative part is orthogonal to the kept part)."""
    A = _sym(H)
    mu = np.trace(A) / A.shape[0]
    lp = orc.eigvalsh_f64(P64)[0]
    ln = orc.eigvalsh_f64(P64 - A)[0]
    ip = np.sum(P64 * (P64 - A)) / (np.linalg.norm(P64) * max(np.linalg.norm(P64 - A), 1e-300))
    return lp / mu, ln / mu, ip


def test_psd_kkt_conditions(orc):
    H = _rand_sym(4, 200)
    H[np.diag_indices(200)] += 4.0
    P, P64 = orc.psd_project(H, 1, return_f64=True)
    lp, ln, ip = _kkt(orc, H, P64)
    assert lp > -1e-12 and ln > -1e-12 and abs(ip) < 1e-12
    w = orc.eigvalsh(H)
    assert np.trace(P64) == pytest.approx(np.maximum(w, 0).sum(), rel=1e-12)
    assert np.linalg.norm(P64 - _sym(H)) == pytest.approx(np.sqrt((np.minimum(w, 0) ** 2).sum()), rel=1e-10)


def test_psd_idempotent(orc):
    H = _rand_sym(5, 160)
    P = orc.psd_project(H)
    PP = orc.psd_project(P)
    assert np.linalg.norm(PP - P) / np.linalg.norm(P) < 1e-6


@pytest.fixture(scope="module")
def stored1024(orc):
    """The stored-Hessian workload at full size: Gram of X = Z L (4096 x 1024),
    packed to Bf16TrilDiagF32 and read back."""
    wl = g.WORKLOADS["stored1024"]
    X = g.x_chunk(wl)
    H32 = orc.gram(X).astype(np.float32)
    Hs = orc.unpack_tril(orc.pack_tril(H32), wl.K)
    P, P64 = orc.psd_project(Hs, 1, return_f64=True)
    return H32, Hs, P, P64


def test_stored_projection_change_below_bf16_step(orc, stored1024):
    gold = json.load(open(os.path.join(GOLD, "pages_values.json")))
    H32, Hs, P, P64 = stored1024
    A = _sym(Hs)
    change = np.linalg.norm(P64 - A) / np.linalg.norm(A)
    assert change < gold["bf16_step_percent"]["value"] / 100.0
    # witness bound: the pre-storage Gram is PSD, so the projection is at least as close
    assert np.linalg.norm(P64 - A) <= np.linalg.norm(H32.astype(np.float64) - A) * (1 + 1e-9)
    lp, ln, ip = _kkt(orc, Hs, P64)
    assert lp > -1e-6 and ln > -1e-9 and abs(ip) < 1e-7


def test_stored_projection_enables_damp_001(orc, stored1024):
    """After projection, Cholesky succeeds at damp 0.01 (dataset card damping table)."""
    H32, Hs, P, P64 = stored1024
    st, U, mu = orc.gptq_U(P, 0.01)
    assert st == orc.OK
