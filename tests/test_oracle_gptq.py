"""CPU pins for the oracle's damping, Cholesky route to U, GPTQ sweep and qerr.

Pages: ork-driver wiki "Exp 2026-08-18 GPTQ Int4" (error-compensated
column-sequential int4 rounding with a Cholesky-based inverse; symmetric codes
in [-8, 7] with per-(row, group) absmax/7 scales, w = code * scale; the qerr
definition and its analytic check on U(-1, 1) weights) and hipfire-calib-data
("The fix": damping in units of mean(diag H); a large damping makes GPTQ
degenerate to round-to-nearest).
"""
import json
import math
import os

import numpy as np
import pytest

import synthgen as g

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _f32(x):
    return np.float32(x)


def _dequant(codes, scales):
    N, K = codes.shape
    G = K // scales.shape[1]
    return (codes.astype(np.float64).reshape(N, -1, G) * scales[:, :, None]).reshape(N, K)


def _gram32(orc, X):
    return orc.gram(X).astype(np.float32)


# ------------------------------------------------------------------ U and Cholesky
def test_cholesky_reconstructs(orc):
    rng = np.random.default_rng(0)
    B = rng.standard_normal((80, 80))
    A = B @ B.T + 80 * np.eye(80)
    st, L = orc.cholesky_lower(A)
    assert st == orc.OK
    assert np.abs(L @ L.T - A).max() < 1e-10 * np.abs(A).max()
    assert np.array_equal(L, np.tril(L))


def test_cholesky_flags_indefinite_and_nan(orc):
    A = np.eye(5); A[4, 4] = -1.0
    assert orc.cholesky_lower(A)[0] == orc.ERR_NOT_PD
    A = np.eye(5); A[2, 2] = np.nan
    assert orc.cholesky_lower(A)[0] == orc.ERR_NOT_PD


def test_U_is_upper_factor_of_damped_inverse(orc):
    wl = g.WORKLOADS["tiny"]
    H = _gram32(orc, g.x_chunk(wl))
    st, U, mu = orc.gptq_U(H, 0.01)
    assert st == orc.OK
    Hd = H.astype(np.float64) + 0.01 * mu * np.eye(wl.K)
    assert mu == pytest.approx(np.trace(H.astype(np.float64)) / wl.K, rel=1e-15)
    assert np.array_equal(U, np.triu(U)) and (np.diag(U) > 0).all()
    assert np.abs(U.T @ U @ Hd - np.eye(wl.K)).max() < 1e-10


def test_U_literal_route_equals_reverse_cholesky_inverse(orc):
    """U = R^{-1} with H_d = R R^T, R upper: an independent route through numpy's
    LAPACK Cholesky and inverse of the order-reversed matrix."""
    rng = np.random.default_rng(1)
    X = rng.standard_normal((200, 60)).astype(np.float32)
    H = _gram32(orc, X)
    st, U, mu = orc.gptq_U(H, 0.01)
    Hd = H.astype(np.float64) + 0.01 * mu * np.eye(60)
    Lr = np.linalg.cholesky(Hd[::-1, ::-1])
    R = Lr[::-1, ::-1]
    np.testing.assert_allclose(U, np.linalg.inv(R), rtol=1e-9, atol=1e-12)


def test_U_lapack_route_equals_plain_route(orc):
    """gptq_U_lapack (the literal route with one LAPACK primitive per step, for
    the largest sizes) against gptq_U's plain loops on a correlated, ill-
    conditioned stored-style Hessian, and the same statuses on bad inputs."""
    wl = g.WORKLOADS["stored1024"]
    X = g.x_chunk(wl, tokens=700)            # T < K: singular before damping
    H = _gram32(orc, X)
    st, U, mu = orc.gptq_U(H, 0.01)
    st2, U2, mu2 = orc.gptq_U_lapack(H, 0.01)
    assert st == st2 == orc.OK and mu == pytest.approx(mu2, rel=1e-14)
    assert np.array_equal(U2, np.triu(U2))
    rel = np.linalg.norm(U2 - U) / np.linalg.norm(U)
    assert rel < 1e-9, rel
    Hn = H.copy(); Hn[5, 3] = np.nan
    assert orc.gptq_U_lapack(Hn, 0.01)[0] == orc.ERR_NONFINITE
    Hu = H.copy(); Hu[3, 5] = np.nan           # upper triangle is never read
    assert orc.gptq_U_lapack(Hu, 0.01)[0] == orc.OK
    assert orc.gptq_U_lapack(np.zeros((8, 8), np.float32), 0.01)[0] == orc.ERR_NO_CALIBRATION
    Hi = np.eye(6, dtype=np.float32); Hi[4, 4] = -3.0
    assert orc.gptq_U_lapack(Hi, 0.01)[0] == orc.ERR_NOT_PD == orc.gptq_U(Hi, 0.01)[0]


# ------------------------------------------------------------------ GPTQ sweep
def _obq_reference(W, H, G, damp):
    """Sequential optimal-brain quantisation with freshly inverted Hessians of the
    not-yet-quantised columns (numpy LAPACK inverse): after column i is rounded,
    the remaining columns F move by -(w_i - q_i) [H_F^{-1}]_{i,:} / [H_F^{-1}]_{ii}.
    GPTQ's Cholesky rows are an exact reformulation of this recursion."""
    W = W.astype(np.float64).copy()
    N, K = W.shape
    Hd = H.astype(np.float64)
    Hd = np.tril(Hd) + np.tril(Hd, -1).T
    Hd = Hd + damp * np.trace(Hd) / K * np.eye(K)
    codes = np.zeros((N, K), np.int8)
    scales = np.zeros((N, K // G), np.float32)
    s = np.zeros(N, np.float32)
    for i in range(K):
        Finv = np.linalg.inv(Hd[i:, i:])
        if i % G == 0:
            s = (np.abs(W[:, i:i + G]).max(1).astype(np.float32) / np.float32(7)).astype(np.float32)
            scales[:, i // G] = s
        v = W[:, i].astype(np.float32) / s
        c = np.clip(np.rint(v), -8, 7)
        codes[:, i] = c
        err = (W[:, i] - c * s.astype(np.float64)) / Finv[0, 0]
        W[:, i:] -= np.outer(err, Finv[0, :])
    return codes, scales


def test_sweep_equals_obq_recursion(orc):
    rng = np.random.default_rng(2)
    N, K, G = 24, 48, 16
    X = (rng.standard_normal((160, 12)) @ rng.standard_normal((12, K)) +
         0.3 * rng.standard_normal((160, K))).astype(np.float32)
    H = _gram32(orc, X)
    W = rng.uniform(-1, 1, (N, K)).astype(np.float32)
    st, codes, scales, _ = orc.gptq(W, H, G, 0.01, want_qerr=False)
    assert st == orc.OK
    rc, rs = _obq_reference(W, H, G, 0.01)
    assert np.array_equal(codes, rc)
    np.testing.assert_allclose(scales, rs, rtol=1e-6)


def test_k2_closed_form(orc):
    """K=2, one group: after rounding column 0, w1' = w1 + (w0 - q0) H01 / (H11 + damp*mu)."""
    H = np.array([[2.0, 0.9], [0.9, 1.5]], np.float32)
    rng = np.random.default_rng(3)
    W = rng.uniform(-1, 1, (200, 2)).astype(np.float32)
    st, codes, scales, _ = orc.gptq(W, H, 2, 0.01, want_qerr=False)
    mu = (2.0 + 1.5) / 2
    for n in range(200):
        s = np.float32(np.float32(max(abs(W[n, 0]), abs(W[n, 1]))) / np.float32(7))
        c0 = int(np.clip(np.rint(np.float32(W[n, 0]) / s), -8, 7))
        w1 = float(W[n, 1]) + (float(W[n, 0]) - c0 * float(s)) * 0.9 / (1.5 + 0.01 * mu)
        c1 = int(np.clip(np.rint(np.float32(w1) / s), -8, 7))
        assert scales[n, 0] == s and codes[n, 0] == c0 and codes[n, 1] == c1


def test_diagonal_hessian_reduces_to_rtn(orc):
    wl = g.WORKLOADS["tiny"]
    W = g.weights(wl).numpy()
    H = _gram32(orc, g.x_chunk(wl))
    Hd = np.diag(np.diag(H)).astype(np.float32)
    st, codes, scales, _ = orc.gptq(W, Hd, wl.group, 0.01)
    rc, rs = orc.rtn(W, wl.group)
    assert st == orc.OK and np.array_equal(codes, rc) and np.array_equal(scales, rs)


def test_power_of_two_scaling_is_bitwise_invariant(orc):
    wl = g.WORKLOADS["tiny"]
    W = g.weights(wl).numpy()
    H = _gram32(orc, g.x_chunk(wl))
    a = orc.gptq(W, H, wl.group, 0.01, imp=np.diag(H).copy())
    b = orc.gptq(W, 4 * H, wl.group, 0.01, imp=np.diag(4 * H).copy())
    assert np.array_equal(a[1], b[1]) and np.array_equal(a[2], b[2]) and a[3] == b[3]


def test_output_error_not_above_rtn(orc):
    """GPTQ minimises ||(W - Q) X||; on the tiny workload it beats round-to-nearest."""
    wl = g.WORKLOADS["tiny"]
    X = g.x_chunk(wl).numpy().astype(np.float64)
    W = g.weights(wl).numpy()
    H = _gram32(orc, X.astype(np.float32))
    st, codes, scales, _ = orc.gptq(W, H, wl.group, wl.damp)
    rc, rs = orc.rtn(W, wl.group)
    e_g = np.linalg.norm((W - _dequant(codes, scales)) @ X.T)
    e_r = np.linalg.norm((W - _dequant(rc, rs)) @ X.T)
    assert e_g <= e_r
    assert codes.min() >= -8 and codes.max() <= 7


def test_rtn_range_and_group_max_exact(orc):
    W = g.uniform_weights(7, 64, 256).numpy()
    codes, scales = orc.rtn(W, 32)
    assert codes.min() >= -7 and codes.max() <= 7        # absmax/7 never needs -8
    # every group's largest-magnitude weight maps to +-7
    a = np.abs(codes.reshape(64, 8, 32)).max(-1)
    assert (a == 7).all()


def test_status_codes(orc):
    wl = g.WORKLOADS["tiny"]
    W = g.weights(wl).numpy()
    H = _gram32(orc, g.x_chunk(wl))
    W2 = W.copy(); W2[3, 7] = np.nan
    assert orc.gptq(W2, H, 32)[0] == orc.ERR_NONFINITE
    H2 = H.copy(); H2[9, 2] = np.inf
    assert orc.gptq(W, H2, 32)[0] == orc.ERR_NONFINITE
    H3 = H.copy(); H3[2, 9] = np.nan                   # upper triangle is never read
    assert orc.gptq(W, H3, 32)[0] == orc.OK
    assert orc.gptq(W, np.zeros_like(H), 32)[0] == orc.ERR_NO_CALIBRATION
    Hi = np.eye(128, dtype=np.float32); Hi[127, 127] = -50.0
    assert orc.gptq(W, Hi, 32)[0] == orc.ERR_NOT_PD
    assert orc.gptq(W, H, 48)[0] == orc.ERR_INVALID_ARG       # K % G != 0
    assert orc.gptq(W[:, :127], H[:127, :127], 127)[0] == orc.ERR_INVALID_ARG   # odd K


def test_pack_codes_layout(orc):
    codes = np.array([[-8, 7, 0, -1, 3, -3]], np.int8)
    packed = orc.pack_codes(codes)
    assert packed.tolist() == [[0x78, 0xF0, 0xD3]]
    assert np.array_equal(orc.unpack_codes(packed, 6), codes)


# ------------------------------------------------------------------ qerr
def _expected_uniform_qerr(G):
    """RTN qerr for U(-1, 1) weights: the group maximum is exact, the other G-1
    errors are uniform over one step s = M/7 with E[M^2] = G/(G+2), so
    qerr = (1/14) sqrt((G-1)/(G+2)); it tends to the wiki's 0.0714 as G grows."""
    return math.sqrt((G - 1) / (G + 2)) / 14.0


def test_qerr_uniform_closed_form(orc):
    gold = json.load(open(os.path.join(GOLD, "pages_values.json")))["qerr_uniform"]
    assert gold["step"] == pytest.approx(1 / 7, abs=1e-4)
    assert gold["rms_quant_error"] == pytest.approx(gold["step"] / math.sqrt(12), abs=1e-5)
    assert gold["rms_w"] == pytest.approx(1 / math.sqrt(3), abs=1e-4)
    assert gold["predicted"] == pytest.approx(gold["rms_quant_error"] / gold["rms_w"], abs=1e-4)
    W = g.uniform_weights(8, 1024, 1024).numpy()         # 2^20 weights
    for G in (32, 128, 1024):
        codes, scales = orc.rtn(W, G)
        q = orc.qerr(codes, scales, W)
        assert q == pytest.approx(_expected_uniform_qerr(G), rel=0.01), G
    codes, scales = orc.rtn(W, 1024)
    assert orc.qerr(codes, scales, W) == pytest.approx(gold["predicted"], rel=0.01)
    # the measured 0.07117 is within 0.4% of the prediction, as the page states
    assert abs(gold["measured"] - gold["predicted"]) / gold["predicted"] < gold["measured_within"]


def test_qerr_importance_properties(orc):
    W = g.uniform_weights(9, 128, 256).numpy()
    codes, scales = orc.rtn(W, 64)
    q1 = orc.qerr(codes, scales, W)
    assert orc.qerr(codes, scales, W, np.ones(256, np.float32)) == q1
    imp = np.exp(np.random.default_rng(0).standard_normal(256)).astype(np.float32)
    qi = orc.qerr(codes, scales, W, imp)
    assert qi != q1                                               # an imatrix moves the value
    assert orc.qerr(codes, scales, W, 4 * imp) == qi              # the scale cancels
    assert orc.qerr(codes, scales, W, imp) == qi                  # deterministic
    q, nd = orc.qerr(codes, scales, W, imp, return_sums=True)
    D = _dequant(codes, scales)
    np.testing.assert_allclose(nd, [(imp * (W - D) ** 2).sum(), (imp * W.astype(np.float64) ** 2).sum()],
                               rtol=1e-12)


def test_qerr_request_leaves_codes_identical(orc):
    wl = g.WORKLOADS["tiny"]
    W = g.weights(wl).numpy()
    H = _gram32(orc, g.x_chunk(wl))
    a = orc.gptq(W, H, 32, want_qerr=True, imp=np.diag(H).copy())
    b = orc.gptq(W, H, 32, want_qerr=False)
    assert np.array_equal(a[1], b[1]) and np.array_equal(a[2], b[2])


# ------------------------------------------------------------------ replay checker
def test_replay_accepts_own_codes_and_flags_wrong_ones(orc):
    wl = g.WORKLOADS["tiny"]
    W = g.weights(wl).numpy()
    H = _gram32(orc, g.x_chunk(wl))
    st, U, mu = orc.gptq_U(H, 0.01)
    codes, scales = orc.gptq_sweep(W, U, 32)
    r = orc.gptq_replay(codes, scales, W, U, 32)
    assert r["exact"] == W.size and r["inadmissible"] == 0 and r["scale_mismatch"] == 0
    bad = codes.copy(); bad[5, 40] = np.clip(bad[5, 40] + 3, -8, 7) if bad[5, 40] < 4 else bad[5, 40] - 3
    r = orc.gptq_replay(bad, scales, W, U, 32)
    assert r["inadmissible"] >= 1
    rc, rs = orc.rtn(W, 32)                         # RTN codes are not GPTQ codes
    assert orc.gptq_replay(rc, rs, W, U, 32)["inadmissible"] > 100


def test_replay_flip_gap_histogram(orc):
    """With a diagonal H (no feedback) and group scale 1, candidate codes that take
    the other neighbour of an exact tie (2.5), of a value 5e-5 of a step from one
    (3.49995) and of a value 5e-4 from one (1.4995) are counted as tie flips in
    the bins [0, 1e-7), [1e-5, 1e-4) and [1e-4, 1e-3); with delta = 1e-4 the last
    one is inadmissible."""
    K, G = 32, 32
    W = np.zeros((1, K), np.float32)
    W[0, 0] = 7.0                                      # scale 7 / 7 = 1
    W[0, 3], W[0, 9], W[0, 20] = 2.5, 3.49995, 1.4995
    U = np.eye(K)
    codes, scales = orc.gptq_sweep(W, U, G)
    assert scales[0, 0] == 1.0 and codes[0, 3] == 2 and codes[0, 9] == 3 and codes[0, 20] == 1
    cand = codes.copy()
    cand[0, 3], cand[0, 9], cand[0, 20] = 3, 4, 2
    r = orc.gptq_replay(cand, scales, W, U, G)
    assert r["tie_flips"] == 3 and r["inadmissible"] == 0
    assert r["flip_gap_hist"] == [1, 0, 0, 1, 1, 0]
    r = orc.gptq_replay(cand, scales, W, U, G, delta=1e-4)
    assert r["tie_flips"] == 2 and r["inadmissible"] == 1
