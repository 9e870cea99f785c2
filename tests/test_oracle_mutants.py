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


def _nf4_qerr_pin_holds(orc):
    """The wiki's NF4 qerr on uniform weights (qerr section, 0.09358)."""
    gold = json.load(open(os.path.join(GOLD, "pages_values.json")))["qerr_nf4"]
    W = g.uniform_weights(8, 256, 1024).numpy()
    codes, scales = orc.rtn(W, 1024, flags=orc.NF4)
    return abs(orc.qerr(codes, scales, W, flags=orc.NF4) - gold["measured"]) / gold["measured"] < 0.01


def _nf4_nearest_pin_holds(orc):
    """NF4 codes are the nearest levels (brute-force argmin), away from midpoints."""
    rng = np.random.default_rng(4)
    W = rng.standard_normal((16, 128)).astype(np.float32)
    codes, scales = orc.rtn(W, 32, flags=orc.NF4)
    L = orc.nf4_levels().astype(np.float64)
    x = (W / np.repeat(scales, 32, axis=1)).astype(np.float32).astype(np.float64)
    d = np.abs(x[..., None] - L)
    srt = np.sort(d, -1)
    clear = srt[..., 1] - srt[..., 0] > 1e-6
    return np.array_equal(codes[clear], d.argmin(-1)[clear])


def _act_perm_pin_holds(orc):
    """Act order's permutation is numpy's stable argsort of the negated diagonal."""
    rng = np.random.default_rng(21)
    X = (rng.standard_normal((100, 40)) * rng.uniform(0.2, 3.0, 40)).astype(np.float32)
    H = orc.gram(X).astype(np.float32)
    return np.array_equal(orc.act_order_perm(H), np.argsort(-np.diag(H), kind="stable"))


def _act_obq_pin_holds(orc):
    """Act order equals OBQ taken in that column order with each column's own group."""
    from test_oracle_variants import _obq_order
    rng = np.random.default_rng(13)
    N, K, G = 20, 48, 16
    X = (rng.standard_normal((160, 12)) @ rng.standard_normal((12, K)) +
         0.3 * rng.standard_normal((160, K))).astype(np.float32)
    X *= rng.uniform(0.3, 3.0, K).astype(np.float32)
    H = orc.gram(X).astype(np.float32)
    H = (np.tril(H) + np.tril(H, -1).T).astype(np.float32)
    W = rng.uniform(-1, 1, (N, K)).astype(np.float32)
    st, codes, scales, _ = orc.gptq(W, H, G, 0.01, want_qerr=False, flags=orc.STATIC_GROUPS | orc.ACT_ORDER)
    rc, rs = _obq_order(W, H, G, 0.01, np.argsort(-np.diag(H), kind="stable"))
    return st == 0 and np.array_equal(codes, rc) and np.array_equal(scales, rs)


def _static_pin_holds(orc):
    """Static scales are the round-to-nearest scales of the original weights."""
    wl = g.WORKLOADS["tiny"]
    W = g.weights(wl).numpy()
    H = orc.gram(g.x_chunk(wl)).astype(np.float32)
    st, codes, scales, _ = orc.gptq(W, H, wl.group, 0.01, flags=orc.STATIC_GROUPS)
    return st == 0 and np.array_equal(scales, orc.rtn(W, wl.group)[1])


PINS = {
    1: _truncation_pin_holds,      # RNE instead of truncation
    2: _sweep_pin_holds,           # error feedback with the wrong sign
    3: _sweep_pin_holds,           # static group scales
    4: _sweep_pin_holds,           # wrong rows of the inverse factor
    5: _psd_pin_holds,             # |lambda| instead of max(lambda, 0)
    6: _qerr_pin_holds,            # importance dropped from the numerator
    7: _gram_pin_holds,            # last token dropped
    8: _index_pin_holds,           # tril row stored reversed
    9: _nf4_qerr_pin_holds,        # NF4 scale absmax/7
    10: _nf4_nearest_pin_holds,    # NF4 rounds down to a level
    11: _act_perm_pin_holds,       # act order ascending
    12: _act_obq_pin_holds,        # act order's groups taken in the permuted order
    13: _static_pin_holds,         # the static switch ignored
}


def test_pins_hold_on_the_real_oracle(orc):
    for n, pin in PINS.items():
        assert pin(orc), n


@pytest.mark.parametrize("n", sorted(PINS))
def test_pin_catches_mutant(mutant, n):
    orc = mutant(n)
    assert not PINS[n](orc)
