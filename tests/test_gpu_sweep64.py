"""GPU parity of gptq_quantize's sweep with its state in fp64 (the default above
K = 8192, forced here at sizes the oracle finishes in seconds) against the CPU
oracle, whose sweep carries its trajectory in fp64 and takes its rounding
decisions in fp32 as the device does.

Bars as for the fp32 sweep (codes identical on >= 99.9% with every difference
a tie flip under the oracle's replay, scales within 1e-5, qerr within 1e-4),
and with the trajectories both in fp64 the codes are expected to agree
outright: the tests also bound the number of tie flips.
"""
import numpy as np
import pytest
import torch

import synthgen as g

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def gq():
    import post_weight_quantization_accumulate_amd as m
    assert torch.cuda.is_available()
    m.lib()
    m.gq_set_sweep_state(m.GQ_SWEEP_F64)
    yield m
    m.gq_set_sweep_state(m.GQ_SWEEP_AUTO)


def _gptq(gq, W, H, G, damp=0.01, imp=None, want_qerr=True):
    N, K = W.shape
    Wt = torch.from_numpy(np.ascontiguousarray(W, np.float32)).to(DEV)
    Ht = torch.from_numpy(np.ascontiguousarray(H, np.float32)).to(DEV)
    it = None if imp is None else torch.from_numpy(np.ascontiguousarray(imp, np.float32)).to(DEV)
    codes = torch.zeros(N, K // 2, dtype=torch.uint8, device=DEV)
    scales = torch.zeros(N, K // G, dtype=torch.float32, device=DEV)
    ws = gq.workspace(gq.gptq_quantize_workspace_size(N, K, G), DEV)
    q = gq.gptq_quantize(codes, scales, Wt, Ht, it, G, damp, ws, want_qerr)
    return codes.cpu().numpy(), scales.cpu().numpy(), q


def _check(orc, W, H, G, codes_packed, scales, q, imp=None, damp=0.01, max_flips=0):
    N, K = W.shape
    st, U, mu = orc.gptq_U(H, damp)
    assert st == orc.OK
    codes = orc.unpack_codes(codes_packed, K)
    oc, os_ = orc.gptq_sweep(W, U, G)
    ident = float((codes == oc).mean())
    rep = orc.gptq_replay(codes, scales, W, U, G)
    print(f"N={N} K={K} G={G}: identity {ident:.6f}, replay {rep}")
    assert rep["inadmissible"] == 0, rep
    assert rep["scale_mismatch"] == 0, rep
    assert rep["tie_flips"] <= max_flips, rep
    assert ident >= 0.999, (ident, rep)
    assert np.allclose(scales, os_, rtol=1e-5, atol=0.0)
    assert codes.min() >= -8 and codes.max() <= 7
    if q is not None:
        qo = orc.qerr(oc, os_, W, imp)
        assert abs(q - qo) / qo < 1e-4
        qg = orc.qerr(codes, scales, W, imp)
        assert abs(q - qg) / qg < 1e-6
    return ident, rep


def test_sweep64_tiny_workload(gq, orc):
    wl = g.WORKLOADS["tiny"]
    W = g.weights(wl).numpy()
    H = orc.gram(g.x_chunk(wl)).astype(np.float32)
    imp = np.diag(H).copy()
    codes, scales, q = _gptq(gq, W, H, wl.group, wl.damp, imp)
    _check(orc, W, H, wl.group, codes, scales, q, imp)


@pytest.mark.parametrize("N,K,G", [(200, 256, 32), (33, 384, 128), (130, 200, 8), (64, 130, 2), (40, 640, 64)])
def test_sweep64_ragged_shapes(gq, orc, N, K, G):
    """Several lazy blocks and groups of 512 columns, a ragged last block
    (200 = 128 + 72, 130 = 128 + 2), rows that do not fill a workgroup."""
    X = g.normal_matrix(N + K, g.S_X, 2 * K, K).numpy()
    mix = g.normal_matrix(N + K, g.S_A, K, K, 1.0 / np.sqrt(K)).numpy()
    X = (X @ (np.eye(K) + mix)).astype(np.float32)
    H = orc.gram(X).astype(np.float32)
    W = g.uniform_weights(N + K, N, K).numpy()
    codes, scales, q = _gptq(gq, W, H, G)
    _check(orc, W, H, G, codes, scales, q)


def test_sweep64_stored_workload_full_size(gq, orc):
    """The stored-Hessian workload (N = K = 1024, G = 128, projected H): the
    fp64 sweep against the oracle, next to the fp32 sweep on the same input."""
    wl = g.WORKLOADS["stored1024"]
    H32 = orc.gram(g.x_chunk(wl)).astype(np.float32)
    P = orc.psd_project(orc.unpack_tril(orc.pack_tril(H32), wl.K))
    W = g.weights(wl).numpy()
    imp = np.diag(H32).copy()
    codes, scales, q = _gptq(gq, W, P, wl.group, wl.damp, imp)
    ident64, rep64 = _check(orc, W, P, wl.group, codes, scales, q, imp, max_flips=2)
    gq.gq_set_sweep_state(gq.GQ_SWEEP_F32)
    try:
        c32, s32, _ = _gptq(gq, W, P, wl.group, wl.damp, imp, want_qerr=False)
    finally:
        gq.gq_set_sweep_state(gq.GQ_SWEEP_F64)
    st, U, mu = orc.gptq_U(P, wl.damp)
    oc, _ = orc.gptq_sweep(W, U, wl.group)
    ident32 = float((orc.unpack_codes(c32, wl.K) == oc).mean())
    print(f"stored1024: fp64 sweep identity {ident64:.6f}, fp32 sweep {ident32:.6f}")
    assert ident64 >= ident32


def _tiny_scale_weights():
    """Groups that need the quotient's exact power-of-two guard: weights around
    1e-30, zeros with one subnormal value, all-subnormal values, and an ordinary
    group beside them."""
    rng = np.random.default_rng(7)
    W = np.zeros((4, 256), np.float32)
    W[:, 0:64] = (rng.uniform(-1, 1, (4, 64)) * 1e-30).astype(np.float32)
    W[:, 64 + 5] = np.float32(3e-39)
    W[1, 64 + 9] = np.float32(-2e-39)
    W[:, 128:192] = (rng.uniform(-1, 1, (4, 64)) * 1e-39).astype(np.float32)
    W[:, 192:256] = rng.uniform(-1, 1, (4, 64)).astype(np.float32)
    return W


@pytest.mark.parametrize("which", ["uniform", "tiny"])
def test_sweep64_diagonal_hessian_is_rtn_bitwise(gq, orc, which):
    """With a diagonal H the sweep feeds no error forward: codes and scales are
    round to nearest's, bit for bit, also where the scale is tiny or
    subnormal (the expected codes checked on the CPU first)."""
    if which == "uniform":
        W = g.uniform_weights(5, 300, 512).numpy()
    else:
        W = _tiny_scale_weights()
        rc, rs = orc.rtn(W, 64)
        assert (rs[:, 1] > 0).all() and (rs[:, 1] < np.float32(1.2e-38)).all()
        assert (rc[:, 64 + 5] == 7).all()
    K = W.shape[1]
    d = np.exp(np.random.default_rng(1).standard_normal(K)).astype(np.float32)
    codes, scales, _ = _gptq(gq, W, np.diag(d), 64, 0.01, want_qerr=False)
    rc, rs = orc.rtn(W, 64)
    assert np.array_equal(scales, rs)
    assert np.array_equal(orc.unpack_codes(codes, K), rc)


def test_sweep64_status_codes(gq, orc):
    wl = g.WORKLOADS["tiny"]
    W = g.weights(wl).numpy()
    H = orc.gram(g.x_chunk(wl)).astype(np.float32)
    W2 = W.copy()
    W2[3, 7] = np.nan
    with pytest.raises(gq.GQError) as e:
        _gptq(gq, W2, H, 32)
    assert e.value.status == gq.GQ_ERR_NONFINITE


def test_sweep_state_setting(gq):
    with pytest.raises(gq.GQError) as e:
        gq.gq_set_sweep_state(7)
    assert e.value.status == gq.GQ_ERR_INVALID_ARG


def _sym_case(N, K, seed):
    X = g.normal_matrix(seed, g.S_X, 2 * K, K).numpy()
    mix = g.normal_matrix(seed, g.S_A, K, K, 1.0 / np.sqrt(K)).numpy()
    X = (X @ (np.eye(K) + mix)).astype(np.float32)
    return g.uniform_weights(seed, N, K).numpy(), X


@pytest.mark.parametrize("N,K,G", [(200, 256, 32), (40, 640, 64), (33, 384, 128)])
def test_split_f64_is_quantize(gq, orc, N, K, G):
    """gptq_factor_f64 + gptq_sweep_f64 are gptq_quantize's fp64 path in two
    halves: the same codes, scales and qerr, bit for bit.  The fp64 U rounds to
    gptq_factor's fp32 U exactly, and matches the oracle's fp64 U (the literal
    route) to 1e-7 relative Frobenius (measured 7e-9: the two routes' fp64
    roundings through H_d's conditioning; fp32's own rounding of U is 3e-8)."""
    W, X = _sym_case(N, K, N + K)
    H = orc.gram(X).astype(np.float32)
    imp = np.diag(H).copy()
    codes, scales, q = _gptq(gq, W, H, G, 0.01, imp)
    Ht = torch.from_numpy(H).to(DEV)
    U64 = torch.empty(K, K, dtype=torch.float64, device=DEV)
    gq.gptq_factor_f64(U64, Ht, 0.01, gq.workspace(gq.gptq_factor_workspace_size(K), DEV))
    U32 = torch.empty(K, K, dtype=torch.float32, device=DEV)
    gq.gptq_factor(U32, Ht, 0.01, gq.workspace(gq.gptq_factor_workspace_size(K), DEV))
    assert torch.equal(U64.to(torch.float32), U32)
    st, Uo, _ = orc.gptq_U(H, 0.01)
    assert st == orc.OK
    Un = U64.cpu().numpy()
    assert np.linalg.norm(Un - Uo) / np.linalg.norm(Uo) < 1e-7
    c2 = torch.empty(N, K // 2, dtype=torch.uint8, device=DEV)
    s2 = torch.empty(N, K // G, dtype=torch.float32, device=DEV)
    q2 = gq.gptq_sweep_f64(c2, s2, torch.from_numpy(W).to(DEV), U64, torch.from_numpy(imp).to(DEV), G,
                           gq.workspace(gq.gptq_sweep_f64_workspace_size(N, K, G), DEV))
    assert np.array_equal(c2.cpu().numpy(), codes) and np.array_equal(s2.cpu().numpy(), scales)
    assert q2 == q


def test_split_f64_argument_errors(gq):
    N, K, G = 8, 64, 32
    W = torch.zeros(N, K, device=DEV)
    U = torch.eye(K, dtype=torch.float64, device=DEV)
    c = torch.empty(N, K // 2, dtype=torch.uint8, device=DEV)
    s = torch.empty(N, K // G, dtype=torch.float32, device=DEV)
    small = gq.workspace(gq.gptq_sweep_f64_workspace_size(N, K, G) - 1024, DEV)
    with pytest.raises(gq.GQError) as e:
        gq.gptq_sweep_f64(c, s, W, U, None, G, small)
    assert e.value.status == gq.GQ_ERR_INVALID_ARG
    s3 = torch.empty(N, K // 3, dtype=torch.float32, device=DEV)        # a group size that is not a power of two
    with pytest.raises(gq.GQError) as e:
        gq.gptq_sweep_f64(c, s3, W, U, None, 3, gq.workspace(gq.gptq_sweep_f64_workspace_size(N, K, G), DEV))
    assert e.value.status == gq.GQ_ERR_INVALID_ARG
