"""Mutation tests: deliberately wrong builds of the oracle (compiled on the CPU
with -DORC_MUTANT=n) must fail the pins that guard them.  This shows each pin
has the power to catch a plausible mistake (the practice of checking that
removing a check makes its test fail, from the hipfire PR #670 write-up).
"""
import json
import os

import numpy as np
import pytest

import synthgen as g

GOLD = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture
def mutant(orc, tmp_path):
    loaded = []

    def use(n):
        orc.use_library(orc.build_mutant(n, str(tmp_path)))
        loaded.append(n)
        return orc
    yield use
    orc.use_library(None)


def _truncation_pin_holds(orc):
    gold = json.load(open(os.path.join(GOLD, "tril_truncation.json")))["vectors"]
    K = len(gold) + 1
    H = np.zeros((K, K), np.float32)
    for n, v in enumerate(gold):
        H.view(np.uint32)[n + 1, 0] = int(v["f32_bits"], 16)
    tril = orc.pack_tril(H)[4 * K:].view(np.uint16)
    return all(tril[(n + 1) * n // 2] == int(v["bf16_bits"], 16) for n, v in enumerate(gold))


def _index_pin_holds(orc):
    K = 9
    H = np.arange(K * K, dtype=np.float32).reshape(K, K) + 1
    tril = orc.pack_tril(H)[4 * K:].view(np.uint16)
    bits = H.view(np.uint32)
    return all(tril[i * (i - 1) // 2 + j] == bits[i, j] >> 16 for i in range(1, K) for j in range(i))


def _gram_pin_holds(orc):
    X = g.normal_matrix(11, g.S_X, 7, 5).numpy()
    H = orc.gram(X)
    ref = X.astype(np.float64).T @ X.astype(np.float64)
    return np.abs(H - ref).max() < 1e-12


def _psd_pin_holds(orc):
    d = np.array([3.0, -1.0, 2.5], np.float32)
    return np.array_equal(orc.psd_project(np.diag(d)), np.diag(np.maximum(d, 0)).astype(np.float32))


def _sweep_pin_holds(orc):
    from test_oracle_gptq import _obq_reference
    rng = np.random.default_rng(2)
    N, K, G = 24, 48, 16
    X = (rng.standard_normal((160, 12)) @ rng.standard_normal((12, K)) +
         0.3 * rng.standard_normal((160, K))).astype(np.float32)
    H = orc.gram(X).astype(np.float32)
    W = rng.uniform(-1, 1, (N, K)).astype(np.float32)
    st, codes, scales, _ = orc.gptq(W, H, G, 0.01, want_qerr=False)
    rc, rs = _obq_reference(W, H, G, 0.01)
    return st == 0 and np.array_equal(codes, rc) and np.allclose(scales, rs, rtol=1e-6)


def _qerr_pin_holds(orc):
    W = g.uniform_weights(9, 16, 64).numpy()
    codes, scales = orc.rtn(W, 16)
    imp = np.exp(np.random.default_rng(0).standard_normal(64)).astype(np.float32)
    q, nd = orc.qerr(codes, scales, W, imp, return_sums=True)
    D = (codes.astype(np.float64).reshape(16, 4, 16) * scales[:, :, None]).reshape(16, 64)
    return np.isclose(nd[0], (imp * (W - D) ** 2).sum(), rtol=1e-12)


PINS = {
    1: _truncation_pin_holds,      # RNE instead of truncation
    2: _sweep_pin_holds,           # error feedback with the wrong sign
    3: _sweep_pin_holds,           # static group scales
    4: _sweep_pin_holds,           # wrong rows of the inverse factor
    5: _psd_pin_holds,             # |lambda| instead of max(lambda, 0)
    6: _qerr_pin_holds,            # importance dropped from the numerator
    7: _gram_pin_holds,            # last token dropped
    8: _index_pin_holds,           # tril row stored reversed
}


def test_pins_hold_on_the_real_oracle(orc):
    for n, pin in PINS.items():
        assert pin(orc), n


@pytest.mark.parametrize("n", sorted(PINS))
def test_pin_catches_mutant(mutant, n):
    orc = mutant(n)
    assert not PINS[n](orc)
