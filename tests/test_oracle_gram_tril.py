"""CPU pins for the oracle's Gram accumulation and Bf16TrilDiagF32 storage.

Pages: hipfire-calib-data dataset card ("Hessian storage: Bf16TrilDiagF32",
"REQUIRED: project to PSD before Cholesky" measurement table) and the AtomicChat
GGUF page ("The importance matrix": the statistic is a sum over chunks).
"""
import json
import os

import numpy as np
import pytest

import synthgen as g

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _bits(x):
    return np.asarray(x, np.float32).view(np.uint32)


# ------------------------------------------------------------------ Gram
def test_gram_brute_force_tiny(orc):
    X = g.normal_matrix(11, g.S_X, 7, 5).numpy()
    H = orc.gram(X)
    for i in range(5):
        for j in range(5):
            ref = 0.0
            for t in range(7):                      # pure-Python sum over tokens
                ref += float(X[t, i]) * float(X[t, j])
            assert H[i, j] == pytest.approx(ref, rel=1e-15, abs=1e-15)


def test_gram_tiny_workload_exact_fp64(orc):
    """fp32 products are exact in fp64, so H differs from the exact rational sum
    only by the fp64 rounding of T additions (bounded by T * 2^-53 * sum|terms|)."""
    wl = g.WORKLOADS["tiny"]
    X = g.x_chunk(wl).numpy()
    H = orc.gram(X)
    assert np.array_equal(H, H.T)
    # exact check on a few entries with Python integers (fp32 = m * 2^e exactly)
    from fractions import Fraction
    for (i, j) in [(0, 0), (5, 3), (127, 0), (64, 63)]:
        terms = [Fraction(float(X[t, i])) * Fraction(float(X[t, j])) for t in range(wl.T)]
        exact = sum(terms)
        bound = sum(abs(x) for x in terms) * wl.T / Fraction(2 ** 53)
        assert abs(Fraction(H[i, j]) - exact) <= bound


def test_gram_diag_is_sum_of_squares(orc):
    """diag(H)[k] = sum_t x_tk^2: the imatrix quantity up to scale (ork-driver wiki,
    GPTQ Int4, qerr paragraph)."""
    X = g.normal_matrix(3, g.S_X, 300, 40).numpy().astype(np.float64)
    H = orc.gram(X.astype(np.float32))
    np.testing.assert_allclose(np.diag(H), (X * X).sum(0), rtol=1e-14)


def test_gram_additive_over_chunks(orc):
    """Accumulating chunk by chunk equals the Gram of the concatenation."""
    X = g.normal_matrix(5, g.S_X, 900, 48).numpy()
    whole = orc.gram(X)
    H = np.zeros((48, 48))
    for a, b in [(0, 128), (128, 500), (500, 900)]:
        orc.gram(X[a:b], H)
    np.testing.assert_allclose(H, whole, rtol=1e-13, atol=1e-12)
    # entries one by one
    I = np.array([0, 47, 13, 20]); J = np.array([0, 3, 13, 47])
    np.testing.assert_allclose(orc.gram_entries(X, I, J), whole[I, J], rtol=1e-13)


def test_gram_cauchy_schwarz_zero_violations(orc):
    """A true Gram matrix has H_ij^2 <= H_ii H_jj for every ordered pair; the
    dataset card reports 0 of 1,047,552 pairs of a 1024 block."""
    gold = json.load(open(os.path.join(GOLD, "pages_values.json")))["cauchy_schwarz_violations"]
    assert gold["pairs"] == 1024 * 1023
    wl = g.WORKLOADS["tiny"]
    H = orc.gram(g.x_chunk(wl)).astype(np.float32).astype(np.float64)
    d = np.diag(H)
    off = ~np.eye(H.shape[0], dtype=bool)
    viol = ((H * H) > np.outer(d, d)) & off
    assert int(viol.sum()) == gold["violations"]


# ------------------------------------------------------------------ tril storage
def test_tril_blob_sizes(orc):
    gold = json.load(open(os.path.join(GOLD, "tril_truncation.json")))
    for K, nbytes in gold["blob_bytes"].items():
        K = int(K)
        assert orc.tril_bytes(K) == nbytes == K * 4 + K * (K - 1) // 2 * 2


def test_tril_truncation_vectors(orc):
    """Golden bit vectors: truncation, not round-to-nearest."""
    gold = json.load(open(os.path.join(GOLD, "tril_truncation.json")))
    vec = gold["vectors"]
    K = len(vec) + 1
    H = np.zeros((K, K), np.float32)
    for n, v in enumerate(vec):              # put vector n at (n+1, 0)
        H.view(np.uint32)[n + 1, 0] = int(v["f32_bits"], 16)
    blob = orc.pack_tril(H)
    tril = blob[4 * K:].view(np.uint16)
    for n, v in enumerate(vec):
        i, j = n + 1, 0
        assert tril[i * (i - 1) // 2 + j] == int(v["bf16_bits"], 16), v


def test_tril_index_and_mirror(orc):
    K = 37
    rng = np.random.default_rng(1)
    H = rng.standard_normal((K, K)).astype(np.float32)
    blob = orc.pack_tril(H)
    diag = blob[:4 * K].view(np.float32)
    tril = blob[4 * K:].view(np.uint16)
    assert np.array_equal(_bits(diag), _bits(np.diag(H)))          # diagonal exact
    for i in range(1, K):
        for j in range(i):
            assert tril[i * (i - 1) // 2 + j] == (_bits(H[i, j]) >> 16)
    Hu = orc.unpack_tril(blob, K)
    assert np.array_equal(_bits(Hu), _bits(Hu.T))                    # mirrored
    low = np.tril_indices(K, -1)
    assert np.array_equal(_bits(Hu)[low], (_bits(H)[low] >> 16) << 16)
    # only the lower triangle is read
    H2 = H.copy(); H2[np.triu_indices(K, 1)] = 123.0
    assert np.array_equal(orc.pack_tril(H2), blob)


def test_tril_roundtrip_bitwise(orc):
    K = 64
    rng = np.random.default_rng(2)
    blob = rng.integers(0, 256, orc.tril_bytes(K), dtype=np.uint8)
    assert np.array_equal(orc.pack_tril(orc.unpack_tril(blob, K)), blob)


def test_stored_gram_keeps_cauchy_schwarz(orc):
    """Truncating off-diagonals towards zero with an exact diagonal cannot create
    a Cauchy-Schwarz violation (the dataset card finds none)."""
    wl = g.WORKLOADS["stored1024"]
    X = g.x_chunk(wl, tokens=512)[:, :256].contiguous()
    H = orc.gram(X).astype(np.float32)
    Hs = orc.unpack_tril(orc.pack_tril(H), 256).astype(np.float64)
    d = np.diag(Hs)
    off = ~np.eye(256, dtype=bool)
    assert int((((Hs * Hs) > np.outer(d, d)) & off).sum()) == 0
