"""GPU parity of the GPTQ variants (gptq_sweep_ex, gptq_quantize_ex,
rtn_quantize_ex) against the oracle, through the C ABI: static groups (scales
fixed before the sweep from the original weights) and the NF4 codebook (scale
absmax, the nearest of 16 levels; the 4-bit pack the ork-driver wiki's qerr
section scores beside the uniform grid).

Round to nearest takes every decision in fp32 on both sides, so codes and scales
are compared bit for bit and qerr to 1e-9.  The sweep variants are held to the
plain sweep's bar: the oracle's replay of the device's decisions finds no
inadmissible code (a code differs only where the oracle's value lies within
1e-3 of a step -- of a midpoint between levels, for NF4 -- from a tie), no scale
off by more than 1e-5 relative, at least 99.9% identical codes, and qerr within
1e-4 of the oracle's.  Static scales equal the oracle's round-to-nearest scales
bit for bit.  Shapes: several tiles, ragged row counts and widths, groups of 2
to 128, an all-zero group under static groups.  Act order (columns by
decreasing diag(H), static groups) is checked on the permuted problem: the
replay runs on W and H permuted by the oracle's permutation, each column with
its original group, over the device's codes put in that order; every decision
must be admissible and 99.9% of them identical given the same history, while
raw identity with the oracle's own run is held to 99% (one legitimate tie flip
on a long row of an ill-conditioned problem moves a few hundred later codes).
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
    return m


def _gpu_rtn(gq, W, G, flags, imp=None):
    N, K = W.shape
    Wd = torch.from_numpy(np.ascontiguousarray(W)).to(DEV)
    codes = torch.empty(N * (K // 2), dtype=torch.uint8, device=DEV)
    scales = torch.empty(N * (K // G), dtype=torch.float32, device=DEV)
    ws = torch.empty(gq.rtn_quantize_workspace_size(N, K, G), dtype=torch.uint8, device=DEV)
    impd = torch.from_numpy(imp).to(DEV) if imp is not None else None
    q = gq.rtn_quantize_ex(codes, scales, Wd, impd, G, flags, ws)
    torch.cuda.synchronize()
    return codes.cpu().numpy().reshape(N, K // 2), scales.cpu().numpy().reshape(N, K // G), q


def _weights(N, K, G, seed):
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((N, K)) * np.exp(0.5 * rng.standard_normal((N, 1)))).astype(np.float32)
    W[0, :G] = 0.0                                   # an all-zero group
    W[rng.integers(0, N, 5), rng.integers(0, K, 5)] = 0.0
    return W


@pytest.mark.parametrize("N,K,G", [(37, 256, 32), (64, 1024, 128), (5, 2048, 8), (9, 64, 1), (9, 64, 2),
                                   (3, 6, 2), (4, 10, 1), (3, 12, 4), (1, 8, 8)])
def test_rtn_nf4_bitexact(gq, orc, N, K, G):
    W = _weights(N, K, G, seed=N * 7 + K + G)
    imp = np.exp(np.random.default_rng(K).standard_normal(K)).astype(np.float32)
    codes, scales, q = _gpu_rtn(gq, W, G, gq.GQ_NF4, imp)
    rc, rs = orc.rtn(W, G, flags=orc.NF4)
    assert np.array_equal(orc.unpack_codes(codes, K, flags=orc.NF4), rc)
    assert np.array_equal(scales, rs)
    assert np.array_equal(codes, orc.pack_codes(rc))
    assert q == pytest.approx(orc.qerr(rc, rs, W, imp, flags=orc.NF4), rel=1e-9, abs=1e-15)
    # the static flag changes nothing for round to nearest
    c2, s2, q2 = _gpu_rtn(gq, W, G, gq.GQ_NF4 | gq.GQ_STATIC_GROUPS, imp)
    assert np.array_equal(c2, codes) and np.array_equal(s2, scales) and q2 == q


def test_rtn_nf4_uniform_weights_qerr(gq, orc):
    """The wiki's NF4 figure on uniform weights (0.09358 measured, 0.0936 in its
    summary), on 2^20 weights in groups of 1024-wide rows cut into 128-groups:
    the device value sits at the closed form sqrt(3 E (G-1)/(G+2)) of the oracle
    test, within 1%, and above the uniform grid's."""
    W = g.uniform_weights(8, 1024, 1024).numpy()
    _, _, q = _gpu_rtn(gq, W, 128, gq.GQ_NF4)
    _, _, qu = _gpu_rtn(gq, W, 128, 0)
    assert 0.0915 < q < 0.0935 and qu < q


def _gpu_gptq(gq, W, H, G, flags, damp=0.01, imp=None, want_qerr=True):
    N, K = W.shape
    Wt = torch.from_numpy(np.ascontiguousarray(W, np.float32)).to(DEV)
    Ht = torch.from_numpy(np.ascontiguousarray(H, np.float32)).to(DEV)
    it = None if imp is None else torch.from_numpy(np.ascontiguousarray(imp, np.float32)).to(DEV)
    codes = torch.zeros(N, K // 2, dtype=torch.uint8, device=DEV)
    scales = torch.zeros(N, K // G, dtype=torch.float32, device=DEV)
    ws = gq.workspace(gq.gptq_quantize_ex_workspace_size(N, K, G, flags), DEV)
    q = gq.gptq_quantize_ex(codes, scales, Wt, Ht, it, G, damp, flags, ws, want_qerr)
    return codes.cpu().numpy(), scales.cpu().numpy(), q


def _check(orc, W, H, G, flags, codes_packed, scales, q, imp=None, damp=0.01):
    N, K = W.shape
    st, U, _ = orc.gptq_U(H, damp)
    assert st == orc.OK
    codes = orc.unpack_codes(codes_packed, K, flags=flags)
    oc, os_ = orc.gptq_sweep(W, U, G, flags=flags)
    ident = float((codes == oc).mean())
    rep = orc.gptq_replay(codes, scales, W, U, G, flags=flags)
    assert rep["inadmissible"] == 0, rep
    assert rep["scale_mismatch"] == 0, rep
    assert ident >= 0.999, (ident, rep)
    if flags & orc.STATIC_GROUPS:
        _, rs = orc.rtn(W, G, flags=flags & orc.NF4)
        assert np.array_equal(scales, rs)
    if flags & orc.NF4:
        assert codes.min() >= 0 and codes.max() <= 15
    else:
        assert codes.min() >= -8 and codes.max() <= 7
    if q is not None:
        qo = orc.qerr(oc, os_, W, imp, flags=flags)
        assert abs(q - qo) / qo < 1e-4
        qg = orc.qerr(codes, scales, W, imp, flags=flags)
        assert abs(q - qg) / qg < 1e-6
    return ident, rep


FLAGS = [1, 2, 3]


@pytest.mark.parametrize("flags", FLAGS)
def test_variant_tiny_workload(gq, orc, flags):
    wl = g.WORKLOADS["tiny"]
    X = g.x_chunk(wl)
    W = g.weights(wl).numpy()
    H = orc.gram(X).astype(np.float32)
    imp = np.diag(H).copy()
    codes, scales, q = _gpu_gptq(gq, W, H, wl.group, flags, wl.damp, imp)
    _check(orc, W, H, wl.group, flags, codes, scales, q, imp)


@pytest.mark.parametrize("flags", FLAGS)
@pytest.mark.parametrize("N,K,G", [(200, 256, 32), (33, 384, 128), (130, 200, 8), (64, 130, 2)])
def test_variant_ragged_shapes(gq, orc, flags, N, K, G):
    X = g.normal_matrix(N + K, g.S_X, 2 * K, K).numpy()
    mix = g.normal_matrix(N + K, g.S_A, K, K, 1.0 / np.sqrt(K)).numpy()
    X = (X @ (np.eye(K) + mix)).astype(np.float32)            # correlated channels
    H = orc.gram(X).astype(np.float32)
    W = g.uniform_weights(N + K, N, K).numpy()
    W[1, G:2 * G] = 0.0                                       # an all-zero group (static: scale 0)
    codes, scales, q = _gpu_gptq(gq, W, H, G, flags)
    _check(orc, W, H, G, flags, codes, scales, q)


def test_sweep_ex_flag_zero_is_the_sweep(gq, orc):
    """gptq_sweep_ex with flags 0 and gptq_sweep give identical bytes, and unknown
    flag bits are refused."""
    wl = g.WORKLOADS["tiny"]
    W = torch.from_numpy(g.weights(wl).numpy()).to(DEV)
    H = torch.from_numpy(orc.gram(g.x_chunk(wl)).astype(np.float32)).to(DEV)
    N, K = W.shape
    G = wl.group
    U = torch.empty(K, K, dtype=torch.float32, device=DEV)
    gq.gptq_factor(U, H, wl.damp, gq.workspace(gq.gptq_factor_workspace_size(K), DEV))
    ws = gq.workspace(gq.gptq_sweep_workspace_size(N, K, G), DEV)
    outs = []
    for ex in (False, True):
        c = torch.zeros(N, K // 2, dtype=torch.uint8, device=DEV)
        s = torch.zeros(N, K // G, dtype=torch.float32, device=DEV)
        q = (gq.gptq_sweep_ex(c, s, W, U, None, G, 0, ws) if ex else gq.gptq_sweep(c, s, W, U, None, G, ws))
        outs.append((c.cpu().numpy(), s.cpu().numpy(), q))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])
    assert outs[0][2] == outs[1][2]
    with pytest.raises(gq.GQError) as e:
        gq.gptq_sweep_ex(c, s, W, U, None, G, 4, ws)
    assert e.value.status == gq.GQ_ERR_INVALID_ARG


def test_nf4_gptq_beats_nf4_rtn_on_output(gq, orc):
    """On correlated activations the NF4 sweep lowers the layer's output error
    tr((W - Q) H (W - Q)^T) below NF4 round to nearest, as the uniform sweep does."""
    K, N, G = 256, 64, 32
    X = g.normal_matrix(5, g.S_X, 4 * K, K).numpy()
    mix = g.normal_matrix(5, g.S_A, K, K, 1.5 / np.sqrt(K)).numpy()
    X = (X @ (np.eye(K) + mix)).astype(np.float32)
    H = orc.gram(X).astype(np.float32)
    W = g.normal_matrix(6, g.S_W, N, K).numpy().astype(np.float32)
    L = orc.nf4_levels().astype(np.float64)

    def deq(cp, s):
        c = orc.unpack_codes(cp, K, flags=orc.NF4)
        return (L[c].reshape(N, -1, G) * s.reshape(N, -1, 1)).reshape(N, K)

    cg, sg, _ = _gpu_gptq(gq, W, H, G, gq.GQ_NF4, want_qerr=False)
    cr, sr, _ = _gpu_rtn(gq, W, G, gq.GQ_NF4)
    H64 = H.astype(np.float64)
    out = lambda Q: float(np.einsum("nk,kl,nl->", W - Q, H64, W - Q))
    assert out(deq(cg, sg)) < 0.9 * out(deq(cr, sr))


def _check_act(orc, W, H, G, flags, codes_packed, scales, q, imp=None, damp=0.01):
    N, K = W.shape
    perm = orc.act_order_perm(H)
    Hs = np.tril(H) + np.tril(H, -1).T
    st, Up, _ = orc.gptq_U(Hs[np.ix_(perm, perm)], damp)
    assert st == orc.OK
    codes = orc.unpack_codes(codes_packed, K, flags=flags)
    st, oc, os_, qo = orc.gptq(W, H, G, damp, imp, want_qerr=q is not None, flags=flags)
    assert st == orc.OK
    ident = float((codes == oc).mean())
    rep = orc.gptq_replay(codes[:, perm], scales, W[:, perm], Up, G, flags=flags & ~orc.ACT_ORDER,
                          gidx=perm // G)
    # every decision admissible, 99.9% identical given the same history; the raw
    # identity with the oracle's own trajectory can lose a few hundred codes to a
    # single legitimate tie flip on a long row (ill-conditioned H, few rows)
    assert rep["inadmissible"] == 0, rep
    assert rep["scale_mismatch"] == 0, rep
    assert rep["exact"] >= 0.999 * codes.size, rep
    assert ident >= 0.99, (ident, rep)
    _, rs = orc.rtn(W, G, flags=flags & orc.NF4)
    assert np.array_equal(scales, rs)                         # static scales, original groups
    if q is not None:
        assert abs(q - qo) / qo < 1e-4
        assert abs(q - orc.qerr(codes, scales, W, imp, flags=flags)) / q < 1e-6
    return ident, rep


def _spread_channels(N, K, seed):
    """Correlated activations with a spread of channel energies (so the
    permutation is far from the identity)."""
    X = g.normal_matrix(seed, g.S_X, 2 * K, K).numpy()
    mix = g.normal_matrix(seed, g.S_A, K, K, 1.0 / np.sqrt(K)).numpy()
    scale = np.exp(g.normal_matrix(seed, g.S_S, 1, K).numpy()[0])
    return ((X @ (np.eye(K) + mix)) * scale).astype(np.float32)


@pytest.mark.parametrize("flags", [5, 7])
@pytest.mark.parametrize("N,K,G", [(200, 256, 32), (33, 384, 128), (130, 200, 8), (64, 130, 2), (40, 1024, 64)])
def test_act_order(gq, orc, flags, N, K, G):
    X = _spread_channels(N, K, N + K)
    H = orc.gram(X).astype(np.float32)
    H = np.tril(H)                                            # the lower triangle is all that is read
    W = g.uniform_weights(N + K, N, K).numpy()
    imp = np.diag(H).copy()
    codes, scales, q = _gpu_gptq(gq, W, H, G, flags, imp=imp)
    _check_act(orc, W, H, G, flags, codes, scales, q, imp)


def test_act_order_argument_errors(gq, orc):
    wl = g.WORKLOADS["tiny"]
    W = torch.from_numpy(g.weights(wl).numpy()).to(DEV)
    H = torch.from_numpy(orc.gram(g.x_chunk(wl)).astype(np.float32)).to(DEV)
    N, K = W.shape
    G = wl.group
    c = torch.zeros(N, K // 2, dtype=torch.uint8, device=DEV)
    s = torch.zeros(N, K // G, dtype=torch.float32, device=DEV)
    big = gq.workspace(gq.gptq_quantize_ex_workspace_size(N, K, G, 5), DEV)
    assert gq.gptq_quantize_ex_workspace_size(N, K, G, 5) > gq.gptq_quantize_workspace_size(N, K, G)
    for flags in (gq.GQ_ACT_ORDER, gq.GQ_ACT_ORDER | gq.GQ_NF4):       # needs static groups
        with pytest.raises(gq.GQError) as e:
            gq.gptq_quantize_ex(c, s, W, H, None, G, wl.damp, flags, big)
        assert e.value.status == gq.GQ_ERR_INVALID_ARG
    small = gq.workspace(gq.gptq_quantize_workspace_size(N, K, G), DEV)
    with pytest.raises(gq.GQError) as e:                                  # act order's workspace is larger
        gq.gptq_quantize_ex(c, s, W, H, None, G, wl.damp, 5, small)
    assert e.value.status == gq.GQ_ERR_INVALID_ARG
    U = torch.empty(K, K, dtype=torch.float32, device=DEV)
    with pytest.raises(gq.GQError) as e:                                  # not through the split sweep
        gq.gptq_sweep_ex(c, s, W, U, None, G, 5, gq.workspace(gq.gptq_sweep_workspace_size(N, K, G), DEV))
    assert e.value.status == gq.GQ_ERR_INVALID_ARG
